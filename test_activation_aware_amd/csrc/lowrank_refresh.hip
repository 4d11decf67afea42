// Online refresh of the rank-16 factors of TTQ for one prompt.
//
// The pages initialise B, A once from the SVD of W and keep them static,
// noting that an online PCA could update them at extra cost (paper-daily.com
// deep reading, section 5, limitations; gist.science French summary,
// section 2B).  The update taken here is one step of subspace iteration toward
// the principal subspace of the activation-weighted weight M = W D^(1/2) (the
// matrix whose error the method's closed form weights, paper-daily.com
// section 2), warm-started from the previous orthonormal right basis V:
//
//   G  = M V             [d_out][16]   (the rank-16 input kernel, W for X)
//   P  = M^T G           [d_in][16]    (partials over row chunks, fp32 MFMA)
//   R  = chol(P^T P)     16 x 16, fp64 (P = V' R, R upper, positive diagonal)
//   V' = P R^-1 (triangular solve per row),  A = V'^T D^(-1/2),  Vs = D^(1/2) V'
//   B  = M V' = W Vs     [d_out][16]   (the rank-16 input kernel again)
//
// after which W_res = fp16(W - B A) is formed by the residual kernel and
// quantised as usual.  Passes over W: G, P and B read it once each (the
// residual reads it a fourth time).
//
// P partial kernel (gfx950 MFMA v_mfma_f32_16x16x4_f32, fp32 in, fp32 out):
// P^T[k][j] = sum_n G[n][k] W[n][j].  A workgroup owns 128 channels and a
// chunk of rows; its 4 waves take interleaved 4-row slices.  Lane l loads
// W[n + l/16][cb + 8 (l%16) .. + 8] (16 bytes, the 16 lanes of a row cover 256
// contiguous bytes) and G[n + l/16][l%16]; MFMA e (e = 0..7) multiplies the
// 16 x 4 slice of G^T by the 4 x 16 slice of W at channels cb + 8 c + e.  The
// 4 waves' sums meet in LDS in wave order; the chunks are added in chunk
// order in fp64 by the next kernel.  Deterministic throughout.
#include "ttq_internal.h"

namespace ttq {

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kR = 16;          // rank
constexpr int kPCols = 128;     // channels per P-partial workgroup
constexpr int kPRows = 512;     // rows per P-partial chunk
constexpr int kPAhead = 8;      // 4-row slices whose loads a wave has in flight
constexpr int kGramCols = 64;   // channels per finalize workgroup

// Vs[k][j] = sqrt(D_j) V[j][k]: the weighted basis in the [16][d_in] layout
// the rank-16 input kernel reads as its A operand
__global__ __launch_bounds__(256) void scale_basis_kernel(int d_in, const float* __restrict__ D,
                                                          const float* __restrict__ V, float* __restrict__ Vs) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d_in) return;
  const float sq = sqrtf(D[j]);
#pragma unroll
  for (int k = 0; k < kR; ++k) Vs[(int64_t)k * d_in + j] = sq * V[(int64_t)j * kR + k];
}

// partial[c][k][j] = sum over rows n of chunk c of G[n][k] W[n][j]
__global__ __launch_bounds__(256) void p_partial_kernel(int d_out, int d_in, const _Float16* __restrict__ W,
                                                        const float* __restrict__ G, float* __restrict__ partial) {
  __shared__ f4 red[4][8][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cb = blockIdx.x * kPCols;
  const int chunk = blockIdx.y;
  const int r0 = chunk * kPRows, r1 = min(d_out, r0 + kPRows);
  const int rl = lane >> 4, cl = lane & 15;
  f4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f4{0.f, 0.f, 0.f, 0.f};
  const _Float16* wp = W + (int64_t)cb + 8 * cl;
  // 4-row slices n = r0 + 4 (wave + 4 i), kPAhead slices' loads in flight
  int n = r0 + 4 * wave;
  for (; n + 16 * (kPAhead - 1) < r1; n += 16 * kPAhead) {
    h8 wa[kPAhead];
    float ga[kPAhead];
#pragma unroll
    for (int u = 0; u < kPAhead; ++u) {
      wa[u] = *reinterpret_cast<const h8*>(wp + (int64_t)(n + 16 * u + rl) * d_in);
      ga[u] = G[(int64_t)(n + 16 * u + rl) * kR + cl];
    }
#pragma unroll
    for (int u = 0; u < kPAhead; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[u], (float)wa[u][e], acc[e], 0, 0, 0);
  }
  for (; n < r1; n += 16) {  // d_out is a multiple of 32: whole 4-row slices
    const h8 wa = *reinterpret_cast<const h8*>(wp + (int64_t)(n + rl) * d_in);
    const float ga = G[(int64_t)(n + rl) * kR + cl];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(ga, (float)wa[e], acc[e], 0, 0, 0);
  }
  // lane l holds P^T[4 (l/16) + i][cb + 8 (l%16) + e]
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][e][lane] = acc[e];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f4 s = red[0][e][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f4 v = red[w][e][lane];
        s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        partial[((int64_t)chunk * kR + 4 * rl + i) * d_in + cb + 8 * cl + e] = s[i];
    }
  }
}

// P[j][k] = sqrt(D_j) * sum over chunks (chunk order, fp64), and this
// workgroup's share of the Gram matrix P^T P over its 64 channels
__global__ __launch_bounds__(256) void p_final_gram_kernel(int d_in, int chunks, const float* __restrict__ D,
                                                           const float* __restrict__ partial, double* __restrict__ P,
                                                           double* __restrict__ gram_part) {
  __shared__ double ps[kGramCols][kR + 1];
  const int t = threadIdx.x;
  const int jl = t & 63, kq = t >> 6;  // channel in block, rank quarter
  const int j = blockIdx.x * kGramCols + jl;
  const double sq = (double)sqrtf(D[j]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = 4 * kq + i;
    double s = 0.0;
    int c = 0;
    for (; c + 8 <= chunks; c += 8) {  // eight chunks' loads in flight, added in chunk order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = partial[((int64_t)(c + u) * kR + k) * d_in + j];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += (double)v[u];
    }
    for (; c < chunks; ++c) s += (double)partial[((int64_t)c * kR + k) * d_in + j];
    const double pv = sq * s;
    ps[jl][k] = pv;
    P[(int64_t)j * kR + k] = pv;
  }
  __syncthreads();
  // 136 distinct entries a <= b, one per thread
  if (t < kR * (kR + 1) / 2) {
    int a = 0, rem = t;
    while (rem >= kR - a) {
      rem -= kR - a;
      ++a;
    }
    const int b = a + rem;
    double s = 0.0;
    for (int q = 0; q < kGramCols; ++q) s += ps[q][a] * ps[q][b];
    gram_part[((int64_t)blockIdx.x * kR + a) * kR + b] = s;
    gram_part[((int64_t)blockIdx.x * kR + b) * kR + a] = s;
  }
}

// Gram = sum of the parts (block order) and its Cholesky factor R (upper,
// R^T R = Gram), fp64 in LDS: thread j < 16 owns column j; step i finishes
// R[i][i] (thread i), then every later column's R[i][j].  A pivot that is
// not positive (a direction P does not span) leaves row i zero.
__global__ __launch_bounds__(256) void cholesky_kernel(int blocks, const double* __restrict__ gram_part,
                                                       double* __restrict__ Rout) {
  __shared__ double g[kR][kR];
  __shared__ double R[kR][kR];
  const int t = threadIdx.x;
  const int a = t >> 4, b = t & 15;
  // (eight parts' loads in flight at a time, added in part order)
  double s = 0.0;
  int q = 0;
  for (; q + 8 <= blocks; q += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = gram_part[((int64_t)(q + u) * kR + a) * kR + b];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; q < blocks; ++q) s += gram_part[((int64_t)q * kR + a) * kR + b];
  g[a][b] = s;
  R[a][b] = 0.0;
  __syncthreads();
  const double floor_ = 1e-30 * (g[0][0] > 0.0 ? g[0][0] : 1.0);
  for (int i = 0; i < kR; ++i) {
    if (t == i) {
      double v = g[i][i];
      for (int m = 0; m < i; ++m) v -= R[m][i] * R[m][i];
      R[i][i] = v > floor_ ? sqrt(v) : 0.0;
    }
    __syncthreads();
    if (t > i && t < kR) {
      double v = g[i][t];
      for (int m = 0; m < i; ++m) v -= R[m][i] * R[m][t];
      R[i][t] = R[i][i] != 0.0 ? v / R[i][i] : 0.0;
    }
    __syncthreads();
  }
  Rout[t] = R[a][b];
}

// V' = P R^-1 by a triangular solve per channel (v R = p, fp64; stored
// fp32), A = V'^T D^(-1/2), Vs = D^(1/2) V'
__global__ __launch_bounds__(256) void apply_kernel(int d_in, const float* __restrict__ D,
                                                    const double* __restrict__ P, const double* __restrict__ Rg,
                                                    float* __restrict__ V, float* __restrict__ A,
                                                    float* __restrict__ Vs) {
  __shared__ double R[kR * kR];
  R[threadIdx.x] = Rg[threadIdx.x];
  __syncthreads();
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d_in) return;
  double p[kR], v[kR];
#pragma unroll
  for (int m = 0; m < kR; ++m) p[m] = P[(int64_t)j * kR + m];
  const double sq = (double)sqrtf(D[j]);
#pragma unroll
  for (int k = 0; k < kR; ++k) {
    double x = p[k];
#pragma unroll
    for (int m = 0; m < k; ++m) x -= v[m] * R[m * kR + k];
    const double rkk = R[k * kR + k];
    v[k] = rkk != 0.0 ? x / rkk : 0.0;
    V[(int64_t)j * kR + k] = (float)v[k];
    A[(int64_t)k * d_in + j] = (float)(v[k] / sq);
    Vs[(int64_t)k * d_in + j] = (float)(v[k] * sq);
  }
}

}  // namespace

size_t lowrank_refresh_ws_bytes(int d_out, int d_in) {
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t chunks = (size_t)(d_out + kPRows - 1) / kPRows;
  const size_t blocks = (size_t)d_in / kGramCols;
  return al((size_t)kR * d_in * 4)                // Vs
         + al((size_t)d_out * kR * 4)             // G
         + al(chunks * kR * (size_t)d_in * 4)     // P partials
         + al((size_t)d_in * kR * 8)              // P
         + al(blocks * kR * kR * 8)               // Gram parts
         + al((size_t)kR * kR * 8);               // R
}

hipError_t launch_lowrank_refresh(int d_out, int d_in, const void* W, const float* D, float* V, float* B,
                                  float* A, void* workspace, hipStream_t s) {
  if (d_in % kPCols != 0 || d_in % kGramCols != 0 || d_out % 32 != 0) return hipErrorInvalidValue;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const int chunks = (d_out + kPRows - 1) / kPRows;
  const int blocks = d_in / kGramCols;
  char* ws = static_cast<char*>(workspace);
  float* Vs = reinterpret_cast<float*>(ws);
  ws += al((size_t)kR * d_in * 4);
  float* G = reinterpret_cast<float*>(ws);
  ws += al((size_t)d_out * kR * 4);
  float* part = reinterpret_cast<float*>(ws);
  ws += al((size_t)chunks * kR * d_in * 4);
  double* P = reinterpret_cast<double*>(ws);
  ws += al((size_t)d_in * kR * 8);
  double* gram = reinterpret_cast<double*>(ws);
  ws += al((size_t)blocks * kR * kR * 8);
  double* Rm = reinterpret_cast<double*>(ws);

  hipLaunchKernelGGL(scale_basis_kernel, dim3((unsigned)((d_in + 255) / 256)), dim3(256), 0, s, d_in, D, V, Vs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // G = W Vs^T: the rank-16 input kernel with W in the place of the input
  e = launch_prescale_z(d_out, d_in, W, false, d_in, nullptr, nullptr, Vs, G, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(p_partial_kernel, dim3((unsigned)(d_in / kPCols), (unsigned)chunks), dim3(256), 0, s, d_out,
                     d_in, static_cast<const _Float16*>(W), G, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(p_final_gram_kernel, dim3((unsigned)blocks), dim3(256), 0, s, d_in, chunks, D, part, P, gram);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(cholesky_kernel, dim3(1), dim3(256), 0, s, blocks, gram, Rm);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(apply_kernel, dim3((unsigned)((d_in + 255) / 256)), dim3(256), 0, s, d_in, D, P, Rm, V, A, Vs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // B = W Vs'^T
  return launch_prescale_z(d_out, d_in, W, false, d_in, nullptr, nullptr, Vs, B, s);
}

}  // namespace ttq
