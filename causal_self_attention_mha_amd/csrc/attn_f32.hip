// fp32 causal attention, forward and backward (fp32 storage and arithmetic,
// no bf16 anywhere).  These kernels serve the fp32 entry points, whose job is
// agreement with the exact result to ~1e-6, not speed: one wavefront per row,
// each lane holding two of the 128 head-dim elements, dot products reduced
// across the wavefront.  Exponentials and logs use the accurate library
// expf/logf.
//
// Math (scaled dot-product attention with causal mask, as called through
// flash_attn_func(q, k, v, causal=True) in the apidog blog "ChatGPTを50ドルで
// 独自にトレーニングする方法", section 5 "Flash Attention integration"):
//   z_ij = s <q_i, k_j> (j <= i),  lse_i = ln sum_j exp(z_ij),
//   o_i = sum_j exp(z_ij - lse_i) v_j
//   delta_i = <dout_i, o_i>,  P_ij = exp(z_ij - lse_i),  dP_ij = <dout_i, v_j>
//   dS_ij = P_ij (dP_ij - delta_i);  dq_i = s sum_j dS_ij k_j;
//   dk_j = s sum_i dS_ij q_i;  dv_j = sum_i P_ij dout_i.
#include "device_common.hpp"
#include "internal.hpp"

namespace na {
namespace {

constexpr int kWaves = 4;  // rows per 256-thread workgroup

__device__ __forceinline__ size_t row_off(int b, int t, int h, int T, int H) {
  return ((static_cast<size_t>(b) * T + t) * H + h) * kHeadDim;
}

// Rows are numbered (b, h, t) with t fastest so neighbouring wavefronts share
// one head's keys in cache.
__device__ __forceinline__ bool decode_row(int T, int H, int B, int& b, int& h, int& t) {
  const long row = static_cast<long>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= static_cast<long>(B) * H * T) return false;
  t = static_cast<int>(row % T);
  const long bh = row / T;
  h = static_cast<int>(bh % H);
  b = static_cast<int>(bh / H);
  return true;
}

__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ v,
                                                      float* __restrict__ o,
                                                      float* __restrict__ lse, int B, int T,
                                                      int H, float scale) {
  int b, h, i;
  if (!decode_row(T, H, B, b, h, i)) return;
  const int lane = threadIdx.x & 63;
  const float2 qi = *reinterpret_cast<const float2*>(q + row_off(b, i, h, T, H) + 2 * lane);
  float m = -INFINITY, l = 0.f;
  float2 acc = make_float2(0.f, 0.f);
  for (int j = 0; j <= i; ++j) {
    const size_t off = row_off(b, j, h, T, H) + 2 * lane;
    const float2 kj = *reinterpret_cast<const float2*>(k + off);
    const float2 vj = *reinterpret_cast<const float2*>(v + off);
    const float z = wave_sum(qi.x * kj.x + qi.y * kj.y) * scale;
    const float m_new = fmaxf(m, z);
    const float alpha = expf(m - m_new);  // 0 on the first key (m = -inf)
    const float p = expf(z - m_new);
    l = l * alpha + p;
    acc.x = acc.x * alpha + p * vj.x;
    acc.y = acc.y * alpha + p * vj.y;
    m = m_new;
  }
  const float inv = 1.f / l;
  *reinterpret_cast<float2*>(o + row_off(b, i, h, T, H) + 2 * lane) =
      make_float2(acc.x * inv, acc.y * inv);
  if (lane == 0) lse[(static_cast<size_t>(b) * H + h) * T + i] = m + logf(l);
}

__global__ __launch_bounds__(256) void delta_f32_kernel(const float* __restrict__ o,
                                                        const float* __restrict__ dout,
                                                        float* __restrict__ delta, int B, int T,
                                                        int H) {
  int b, h, i;
  if (!decode_row(T, H, B, b, h, i)) return;
  const int lane = threadIdx.x & 63;
  const size_t off = row_off(b, i, h, T, H) + 2 * lane;
  const float2 oi = *reinterpret_cast<const float2*>(o + off);
  const float2 gi = *reinterpret_cast<const float2*>(dout + off);
  const float d = wave_sum(oi.x * gi.x + oi.y * gi.y);
  if (lane == 0) delta[(static_cast<size_t>(b) * H + h) * T + i] = d;
}

// One wavefront per key row j: loops over the queries i >= j that see it.
__global__ __launch_bounds__(256) void dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv, int B,
    int T, int H, float scale) {
  int b, h, j;
  if (!decode_row(T, H, B, b, h, j)) return;
  const int lane = threadIdx.x & 63;
  const size_t offj = row_off(b, j, h, T, H) + 2 * lane;
  const float2 kj = *reinterpret_cast<const float2*>(k + offj);
  const float2 vj = *reinterpret_cast<const float2*>(v + offj);
  const float* lse_bh = lse + (static_cast<size_t>(b) * H + h) * T;
  const float* del_bh = delta + (static_cast<size_t>(b) * H + h) * T;
  float2 gk = make_float2(0.f, 0.f), gv = make_float2(0.f, 0.f);
  for (int i = j; i < T; ++i) {
    const size_t offi = row_off(b, i, h, T, H) + 2 * lane;
    const float2 qi = *reinterpret_cast<const float2*>(q + offi);
    const float2 gi = *reinterpret_cast<const float2*>(dout + offi);
    const float z = wave_sum(qi.x * kj.x + qi.y * kj.y) * scale;
    const float dp = wave_sum(gi.x * vj.x + gi.y * vj.y);
    const float p = expf(z - lse_bh[i]);
    const float ds = p * (dp - del_bh[i]);
    gv.x += p * gi.x;
    gv.y += p * gi.y;
    gk.x += ds * qi.x;
    gk.y += ds * qi.y;
  }
  *reinterpret_cast<float2*>(dk + offj) = make_float2(gk.x * scale, gk.y * scale);
  *reinterpret_cast<float2*>(dv + offj) = gv;
}

// One wavefront per query row i: loops over the keys j <= i it sees.
__global__ __launch_bounds__(256) void dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dq, int B, int T, int H, float scale) {
  int b, h, i;
  if (!decode_row(T, H, B, b, h, i)) return;
  const int lane = threadIdx.x & 63;
  const size_t offi = row_off(b, i, h, T, H) + 2 * lane;
  const float2 qi = *reinterpret_cast<const float2*>(q + offi);
  const float2 gi = *reinterpret_cast<const float2*>(dout + offi);
  const float lse_i = lse[(static_cast<size_t>(b) * H + h) * T + i];
  const float del_i = delta[(static_cast<size_t>(b) * H + h) * T + i];
  float2 acc = make_float2(0.f, 0.f);
  for (int j = 0; j <= i; ++j) {
    const size_t offj = row_off(b, j, h, T, H) + 2 * lane;
    const float2 kj = *reinterpret_cast<const float2*>(k + offj);
    const float2 vj = *reinterpret_cast<const float2*>(v + offj);
    const float z = wave_sum(qi.x * kj.x + qi.y * kj.y) * scale;
    const float dp = wave_sum(gi.x * vj.x + gi.y * vj.y);
    const float ds = expf(z - lse_i) * (dp - del_i);
    acc.x += ds * kj.x;
    acc.y += ds * kj.y;
  }
  *reinterpret_cast<float2*>(dq + offi) = make_float2(acc.x * scale, acc.y * scale);
}

inline dim3 row_grid(int B, int T, int H) {
  const long rows = static_cast<long>(B) * H * T;
  return dim3(static_cast<unsigned>((rows + kWaves - 1) / kWaves));
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int T, int H, hipStream_t s) {
  const float scale = 1.0f / sqrtf(static_cast<float>(kHeadDim));
  return launch(fwd_f32_kernel, row_grid(B, T, H), dim3(256), 0, s, q, k, v, o, lse, B, T, H,
                scale);
}

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* delta, int B, int T, int H, hipStream_t s) {
  const float scale = 1.0f / sqrtf(static_cast<float>(kHeadDim));
  const dim3 g = row_grid(B, T, H);
  hipError_t e = launch(delta_f32_kernel, g, dim3(256), 0, s, o, dout, delta, B, T, H);
  if (e != hipSuccess) return e;
  e = launch(dkdv_f32_kernel, g, dim3(256), 0, s, q, k, v, dout, lse, delta, dk, dv, B, T, H,
             scale);
  if (e != hipSuccess) return e;
  return launch(dq_f32_kernel, g, dim3(256), 0, s, q, k, v, dout, lse, delta, dq, B, T, H, scale);
}

}  // namespace na
