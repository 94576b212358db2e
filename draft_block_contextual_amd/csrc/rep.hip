// Row LayerNorm and pair-state assembly of the representation stage (review
// of arXiv 2610.12570, "Contextual Correction of Parallel Drafts for
// Speculative Decoding", part 1 of "New approach: DCOCO", paper Sec. 3.2):
//   g_i     = LN(P_h h_i),  b_{i,k} = LN(P_e E[c_{i,k}])   (non-affine LN)
//   s_p     = W_pair [h_p; h_{p+1}] = W_L h_p + W_R h_{p+1}
// The projections arrive as fp32 split-K partial sums, added here in a fixed
// order.  LN statistics are two-pass in fp32 (mean, then mean of squared
// deviations), one wave64 per row.
#include "common.h"
#include "kernels.h"

namespace dcoco {

namespace {

template <typename TO, int VPL>
__global__ void __launch_bounds__(256)
ln_rows_kernel(const float* __restrict__ x, int split, int M, int ldx, int col0, int r, float eps,
               TO* __restrict__ y) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane_id();
  if (row >= M) return;
  float v[VPL];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = l + i * kWave;
    float a = 0.f;
    if (c < r) {
      for (int s = 0; s < split; ++s)
        a += x[(static_cast<long long>(s) * M + row) * ldx + col0 + c];
    }
    v[i] = a;
    sum += a;
  }
  const float mean = wave_sum(sum) / static_cast<float>(r);
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = l + i * kWave;
    v[i] = c < r ? v[i] - mean : 0.f;
    sq += v[i] * v[i];
  }
  const float var = wave_sum(sq) / static_cast<float>(r);
  const float inv = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = l + i * kWave;
    if (c < r) y[static_cast<long long>(row) * r + c] = Elem<TO>::from_f32(v[i] * inv);
  }
}

__global__ void __launch_bounds__(256)
pair_state_kernel(const float* __restrict__ Y, int split, int N, int B, int ldy, int cl, int cr,
                  int rs, float* __restrict__ s) {
  const long long total = static_cast<long long>(N) * (B - 1) * rs;
  const long long M = static_cast<long long>(N) * B;
  for (long long t = blockIdx.x * 256ll + threadIdx.x; t < total; t += 256ll * gridDim.x) {
    const int j = static_cast<int>(t % rs);
    const long long np = t / rs;
    const long long n = np / (B - 1);
    const long long p = np % (B - 1);
    const long long rl = n * B + p;
    float left = 0.f, right = 0.f;
    for (int q = 0; q < split; ++q) {
      left += Y[(q * M + rl) * ldy + cl + j];
      right += Y[(q * M + rl + 1) * ldy + cr + j];
    }
    s[t] = left + right;
  }
}

template <typename TO>
hipError_t launch_ln_t(const float* x, int split, int M, int ldx, int col0, int r, float eps, void* y,
                       hipStream_t st) {
  dim3 grid((M + 3) / 4);
  TO* yo = static_cast<TO*>(y);
  const int vpl = (r + kWave - 1) / kWave;
#define DCOCO_LN(V) hipLaunchKernelGGL((ln_rows_kernel<TO, V>), grid, dim3(256), 0, st, x, split, M, ldx, col0, r, eps, yo)
  if (vpl <= 1) DCOCO_LN(1);
  else if (vpl <= 2) DCOCO_LN(2);
  else if (vpl <= 4) DCOCO_LN(4);
  else if (vpl <= 8) DCOCO_LN(8);
  else if (vpl <= 16) DCOCO_LN(16);
  else DCOCO_LN(32);
#undef DCOCO_LN
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ln_rows(const float* x, int split, int M, int ldx, int col0, int r, float eps,
                          void* y, int out_dtype, hipStream_t st) {
  if (out_dtype == kDtypeBf16) return launch_ln_t<bf16>(x, split, M, ldx, col0, r, eps, y, st);
  return launch_ln_t<float>(x, split, M, ldx, col0, r, eps, y, st);
}

hipError_t launch_pair_state(const float* Y, int split, int N, int B, int ldy, int cl, int cr,
                             int rs, float* s, hipStream_t st) {
  const long long total = static_cast<long long>(N) * (B - 1) * rs;
  if (total <= 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  dim3 grid(static_cast<unsigned>(blocks < 65535 ? blocks : 65535));
  hipLaunchKernelGGL(pair_state_kernel, grid, dim3(256), 0, st, Y, split, N, B, ldy, cl, cr, rs, s);
  return hipGetLastError();
}

}  // namespace dcoco
