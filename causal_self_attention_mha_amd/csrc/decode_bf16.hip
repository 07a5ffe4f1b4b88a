// bf16 single-token decode over a ragged, padded KV cache (split-KV).
//
// Per (b, h), with L = seqlens[b] clamped to [0, T_cap]:
//   z_j = s <q_bh, K[b, j, h]>  (j < L),  o = softmax(z) V[b, 0:L, h],
//   lse = ln sum_j exp(z_j)
// i.e. the attention step nanochat's inference engine runs per generated
// token against its prefilled prompt cache through flash_attn_with_kvcache
// (apidog blog "ChatGPTを50ドルで独自にトレーニングする方法", section 6
// "inference engine"); the new token's key and value are already in the cache
// at row L-1.
//
// The work is HBM bound (each cached K and V byte is used once).  Two kernels:
//   split:   one workgroup per (chunk of 256 keys, h, b) with keys < L; pass 1
//            streams the chunk's K rows (16 lanes x 16 B per 256-byte head row)
//            into scores in LDS, then the chunk max and exponentials, pass 2
//            streams V and accumulates; writes unnormalised o_c, m_c, l_c.
//   combine: one workgroup per (b, h): o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
// Rows t >= L are never read.
#include "device_common.hpp"
#include "internal.hpp"

namespace na {
namespace {

constexpr int D = kHeadDim;
constexpr int CHUNK = 256;  // keys per split workgroup

__host__ __device__ inline int n_chunks(int T_cap) { return (T_cap + CHUNK - 1) / CHUNK; }

// workspace: o_part [B][NC][H][D] fp32, then ml [B][NC][H][2] fp32 (m_c, l_c)
__global__ __launch_bounds__(256) void decode_split_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kc, const u16* __restrict__ vc,
    const int* __restrict__ seqlens, float* __restrict__ opart, float* __restrict__ ml, int B,
    int H, int T_cap, float scale) {
  __shared__ float zs[CHUNK];
  __shared__ float red[8];
  __shared__ __attribute__((aligned(16))) float part[16][D];

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int NC = gridDim.x;
  const int L = min(max(seqlens[b], 0), T_cap);
  const int j0 = c * CHUNK;
  if (j0 >= L) return;  // uniform across the workgroup
  const int n = min(CHUNK, L - j0);

  const int tid = threadIdx.x;
  const int grp = tid >> 4;    // which key of a 16-key pass
  const int chunk = tid & 15;  // which 8 elements of the head row
  const size_t rs = static_cast<size_t>(H) * D;
  const size_t base = static_cast<size_t>(b) * T_cap * rs + static_cast<size_t>(h) * D +
                      8 * chunk;

  float qv[8];
  {
    const uint4 x = ld16(q + (static_cast<size_t>(b) * H + h) * D + 8 * chunk);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t u = (&x.x)[w];
      qv[2 * w] = __uint_as_float(u << 16) * scale;
      qv[2 * w + 1] = __uint_as_float(u & 0xffff0000u) * scale;
    }
  }

  // pass 1: scores
#pragma unroll 4
  for (int p = 0; p < CHUNK / 16; ++p) {
    const int j = p * 16 + grp;
    float acc = 0.f;
    if (j < n) {
      const uint4 x = ld16(kc + base + static_cast<size_t>(j0 + j) * rs);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = (&x.x)[w];
        acc = fmaf(qv[2 * w], __uint_as_float(u << 16), acc);
        acc = fmaf(qv[2 * w + 1], __uint_as_float(u & 0xffff0000u), acc);
      }
    }
    acc = sum16(acc);
    if (chunk == 0) zs[j] = j < n ? acc : -INFINITY;
  }
  __syncthreads();

  // chunk max and exponentials (one score per thread)
  const float z = zs[tid];
  float mx = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float e = expf(z - m);  // 0 for the -inf tail
  float sum = wave_sum(e);
  __syncthreads();  // red[] reads done before reuse
  zs[tid] = e;
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = sum;
  __syncthreads();

  // pass 2: o_c = sum_j e_j V_j over this thread's keys, then across groups
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int p = 0; p < CHUNK / 16; ++p) {
    const int j = p * 16 + grp;
    if (j < n) {
      const float w8 = zs[j];
      const uint4 x = ld16(vc + base + static_cast<size_t>(j0 + j) * rs);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = (&x.x)[w];
        acc[2 * w] = fmaf(w8, __uint_as_float(u << 16), acc[2 * w]);
        acc[2 * w + 1] = fmaf(w8, __uint_as_float(u & 0xffff0000u), acc[2 * w + 1]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[grp][8 * chunk + i] = acc[i];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) s += part[g][tid];
    const size_t slot = (static_cast<size_t>(b) * NC + c) * H + h;
    opart[slot * D + tid] = s;
    if (tid == 0) {
      ml[2 * slot] = m;
      ml[2 * slot + 1] = red[4] + red[5] + red[6] + red[7];
    }
  }
}

__global__ __launch_bounds__(128) void decode_combine_kernel(
    const float* __restrict__ opart, const float* __restrict__ ml,
    const int* __restrict__ seqlens, u16* __restrict__ o, float* __restrict__ lse, int H,
    int T_cap, int NC) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(max(seqlens[b], 0), T_cap);
  const int nc = (L + CHUNK - 1) / CHUNK;
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c)
    M = fmaxf(M, ml[2 * ((static_cast<size_t>(b) * NC + c) * H + h)]);
  float den = 0.f, num = 0.f;
  for (int c = 0; c < nc; ++c) {
    const size_t slot = (static_cast<size_t>(b) * NC + c) * H + h;
    const float w = expf(ml[2 * slot] - M);
    den = fmaf(w, ml[2 * slot + 1], den);
    num = fmaf(w, opart[slot * D + d], num);
  }
  const float out = nc > 0 ? num / den : 0.f;
  o[(static_cast<size_t>(b) * H + h) * D + d] = __builtin_bit_cast(u16, to_bf16(out));
  if (lse != nullptr && d == 0)
    lse[static_cast<size_t>(b) * H + h] = nc > 0 ? M + logf(den) : -INFINITY;
}

}  // namespace

std::size_t decode_workspace_bytes(int B, int H, int T_cap) {
  const std::size_t slots = static_cast<std::size_t>(B) * n_chunks(T_cap) * H;
  return slots * (D + 2) * sizeof(float);
}

hipError_t launch_decode_bf16(const void* q, const void* kc, const void* vc, const int* seqlens,
                              void* o, float* lse, int B, int H, int T_cap, void* ws,
                              hipStream_t s, hipEvent_t const* ev) {
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const int NC = n_chunks(T_cap);
  float* opart = static_cast<float*>(ws);
  float* ml = opart + static_cast<std::size_t>(B) * NC * H * D;
  hipError_t e = mark(ev, 0, s);
  if (e != hipSuccess) return e;
  e = launch(decode_split_kernel, dim3(NC, H, B), dim3(256), 0, s,
                        static_cast<const u16*>(q), static_cast<const u16*>(kc),
                        static_cast<const u16*>(vc), seqlens, opart, ml, B, H, T_cap, scale);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, 1, s)) != hipSuccess) return e;
  e = launch(decode_combine_kernel, dim3(H, B), dim3(128), 0, s, static_cast<const float*>(opart),
             static_cast<const float*>(ml), seqlens, static_cast<u16*>(o), lse, H, T_cap, NC);
  if (e != hipSuccess) return e;
  return mark(ev, 2, s);
}

}  // namespace na
