// bf16 single-token decode over a ragged, padded KV cache (split-KV).
//
// Per (b, h), with L = seqlens[b] clamped to [0, T_cap] and j0 = 0 (or, with
// a sliding window W, j0 = max(0, L - 1 - W): the query sits at row L - 1):
//   z_j = s <q_bh, K[b, j, h]>  (j0 <= j < L),  o = softmax(z) V[b, j0:L, h],
//   lse = ln sum_j exp(z_j)
// i.e. the attention step nanochat's inference engine runs per generated
// token against its prefilled prompt cache through flash_attn_with_kvcache
// (apidog blog "ChatGPTを50ドルで独自にトレーニングする方法", section 6
// "inference engine"); the new token's key and value are already in the cache
// at row L-1.
//
// The work is HBM bound (each cached K and V byte is used once).  Two kernels:
//   split:   persistent workgroups, all heads per workgroup, one 16-lane
//            group per head reading whole 256-byte head rows.  The visible
//            keys of all sequences, laid end to end, are cut into P equal
//            contiguous ranges (P workgroups, at least KMIN keys each), so
//            every workgroup streams the same number of rows whatever the
//            lengths; a range may span several sequences and each sequence
//            is covered by a few consecutive ranges.  Each group streams its
//            range in batches of U keys with an online softmax in registers;
//            the next batch's K and V loads (possibly the next sequence's,
//            with its query) are in flight while the current batch is
//            computed.  For every (sequence, range) segment it writes the
//            unnormalised o_s and (m_s, l_s) per head, and the workgroup that
//            ends a sequence writes its segment count.
//   combine: one 64-thread workgroup per (b, h) (two elements per thread), one
//            pass with a running max over the sequence's segments:
//            o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
// Equal ranges matter: one workgroup per fixed-size chunk leaves the last
// chunks of the longest sequences running on a few compute units while the
// rest of the chip idles.  Rows t >= L (and, with a window, rows before j0)
// are never read.  With H_kv key/value heads the cache is (B, T_cap, H_kv, D)
// and query head h reads head h / (H / H_kv); with 2 or 4 query heads per
// key/value head one 16-lane group loads each row of its key/value head once
// and scores it against all of them.
#include <algorithm>
#include <climits>
#include <mutex>

#include "device_common.hpp"
#include "internal.hpp"

#ifndef NA_DECODE_U
#define NA_DECODE_U 4
#endif
#ifndef NA_DECODE_WG_PER_CU
#define NA_DECODE_WG_PER_CU 2
#endif
#ifndef NA_DECODE_NT
#define NA_DECODE_NT 1
#endif
#ifndef NA_DECODE_WG_PER_CU_GROUPED
#define NA_DECODE_WG_PER_CU_GROUPED 4
#endif

namespace na {
namespace {

constexpr int D = kHeadDim;
constexpr int KMIN = 64;         // fewest keys in a workgroup's range
constexpr int U = NA_DECODE_U;  // keys per batch (per 16-lane group)
constexpr int kWgPerCu = NA_DECODE_WG_PER_CU;  // persistent workgroups per compute unit
constexpr int kWgPerCuGrouped = NA_DECODE_WG_PER_CU_GROUPED;  // the same with grouped heads
constexpr int kMaxB = 4096;      // sequences per split/combine launch pair

// Cached rows are read once, so they stream with non-temporal loads (which do
// not displace reusable lines from the caches): 68.3 -> 61.2 us per d20 call,
// against a plain read of the same bytes at 6.6 TB/s with such loads.
// NA_DECODE_U, NA_DECODE_WG_PER_CU and NA_DECODE_NT are build-time tunables.
__device__ __forceinline__ uint4 ld_row(const u16* p) {
#if NA_DECODE_NT
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return ld16(p);
#endif
}

// Segments per sequence at most: ranges hold at least KMIN keys, so L <= T_cap
// visible keys meet at most ceil((L - 1) / KMIN) + 1 of them.
__host__ __device__ inline int seg_cap(int T_cap) { return (T_cap + KMIN - 1) / KMIN + 1; }

// Sequences per launch pair: at most kMaxB, and few enough that the prefix
// sums of the visible key counts (at most T_cap each) fit an int.
inline int batch_cap(int T_cap) { return std::max(1, std::min(kMaxB, INT_MAX / std::max(T_cap, 1))); }

// workspace: o_part [Bs][SC][H][D] fp32, then ml [Bs][SC][H][2] fp32 (m_s, l_s),
// then nseg [Bs] int32, with Bs = min(B, batch_cap(T_cap)), SC = seg_cap(T_cap)
//
// Persistent split: a workgroup of 16 H threads (one 16-lane group per head,
// lane i of a group owns bytes 16 i .. 16 i + 15 of the 256-byte head row).
// With n_b visible keys in sequence b and pre[b] = n_0 + ... + n_{b-1}, the
// flattened key x = pre[b] + r is row j0_b + r of sequence b, and workgroup w
// of P takes x in [floor(w N / P), floor((w + 1) N / P)), N = pre[B].
struct Batch {
  int b;     // sequence, or -1 past the end of the range
  int j;     // first cache row of the batch
  int jend;  // end of the segment's rows (rows j .. min(j + U, jend) - 1 are used)
};

// GQ: query heads per 16-lane group.  GQ = 1: one group per query head (any
// H / H_kv).  GQ = H / H_kv > 1: one group per key/value head, which loads
// each cached row once and scores it against all GQ query heads that read it.
template <int GQ>
__global__ __launch_bounds__(512) void decode_split_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kc, const u16* __restrict__ vc,
    const int* __restrict__ seqlens, float* __restrict__ opart, float* __restrict__ ml,
    int* __restrict__ nseg, int B, int H, int Hk, int T_cap, float scale, int win, int app,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, float eps) {
  __shared__ int pre[kMaxB + 1];  // pre[b] = visible keys of sequences < b
  const int tid = threadIdx.x;
  const int gi = tid >> 4;  // 16-lane group
  const int l16 = tid & 15;
  const int SC = seg_cap(T_cap);
  // app = 1: the new token was just appended at row seqlens[b] (clamped to
  // T_cap - 1), which the sequence now includes
  auto len = [&](int b) { return min(max(seqlens[b], 0), T_cap - app) + app; };
  // first visible key of a sequence of length L (win < 0: no window)
  auto first_key = [&](int L) { return win < 0 ? 0 : max(0, L - 1 - win); };
  {
    // prefix sums of the visible key counts: serial over blocks of SW
    // sequences, each block summed by the first SW threads (SW: a power of
    // two no larger than the workgroup, which may have only 16 threads)
    const int SW = blockDim.x >= 64 ? 64 : blockDim.x >= 32 ? 32 : 16;
    if (tid < SW) {
      int run = 0;
      for (int b0 = 0; b0 < B; b0 += SW) {
        const int b = b0 + tid;
        int x = 0;
        if (b < B) {
          const int L = len(b);
          x = L - first_key(L);
        }
        for (int o = 1; o < SW; o <<= 1) {  // inclusive scan over SW lanes
          const int y = __shfl_up(x, o, SW);
          if (tid >= o) x += y;
        }
        if (b < B) pre[b + 1] = run + x;
        run += __shfl(x, SW - 1, SW);
      }
      if (tid == 0) pre[0] = 0;
    }
    __syncthreads();
  }
  const int N = pre[B];
  // effective workgroup count: at least KMIN keys per range (one range when
  // N < KMIN); the workgroups past it have no work
  const int P = max(1, min(static_cast<int>(gridDim.x), N / KMIN));
  const int w = blockIdx.x;
  if (N == 0 || w >= P) return;  // uniform over the workgroup
  const int x_lo = static_cast<int>(static_cast<long>(w) * N / P);
  const int x_hi = static_cast<int>(static_cast<long>(w + 1) * N / P);
  // the workgroup whose range holds flattened key x
  auto owner = [&](int x) {
    return static_cast<int>((static_cast<long>(x + 1) * P - 1) / N);
  };
  // the segment that starts at flattened key x < x_hi: the sequence holding x
  // (largest b with pre[b] <= x, which has pre[b + 1] > x) and its rows
  auto segment = [&](int x) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= x) lo = mid; else hi = mid - 1;
    }
    const int j0 = first_key(len(lo));
    return Batch{lo, j0 + x - pre[lo], j0 + min(x_hi, pre[lo + 1]) - pre[lo]};
  };
  auto next = [&](const Batch& t) {
    if (t.j + U < t.jend) return Batch{t.b, t.j + U, t.jend};
    const int x = pre[t.b + 1] < x_hi ? pre[t.b + 1] : x_hi;  // flattened end of the segment
    return x < x_hi ? segment(x) : Batch{-1, 0, 0};
  };

  // the cache has Hk key/value heads; query head h reads head h / (H / Hk);
  // this group serves query heads h0 .. h0 + GQ - 1
  const int hk = GQ == 1 ? gi / (H / Hk) : gi;
  const int h0 = GQ == 1 ? gi : gi * GQ;
  const size_t rs = static_cast<size_t>(Hk) * D;
  const float c2 = scale * 1.4426950408889634f;  // scores in the exp2 domain
  auto rows = [&](const Batch& t, uint4 (&xk)[U], uint4 (&xv)[U]) {
    const size_t base = static_cast<size_t>(t.b) * T_cap * rs + static_cast<size_t>(hk) * D +
                        8 * l16;
    const int rsi = Hk * D;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      // rows past the segment's end: its last row is read again instead
      // (zero weight), so no row outside the visible keys is read
      const size_t r = static_cast<size_t>(min(t.j + i, t.jend - 1)) * rsi;
      xk[i] = ld_row(kc + base + r);
      xv[i] = ld_row(vc + base + r);
    }
  };
  struct QRows {
    uint4 x[GQ];
  };
  auto qrow = [&](const Batch& t) {
    QRows r;
#pragma unroll
    for (int g = 0; g < GQ; ++g)
      r.x[g] = ld16(q + (static_cast<size_t>(t.b) * H + h0 + g) * D + 8 * l16);
    return r;
  };

  float qv[GQ][8];
  // cos_t non-null: the query rows are raw heads, RMS-normalised and rotated
  // at the query's position L - 1 here (the lane holds elements 8 l16 .. + 7;
  // the pair partner of element i < 64 is 8 lanes away)
  auto set_q = [&](const QRows& r, int b) {
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      float x[8];
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        const uint32_t u = (&r.x[g].x)[w4];
        x[2 * w4] = __uint_as_float(u << 16);
        x[2 * w4 + 1] = __uint_as_float(u & 0xffff0000u);
      }
      if (cos_t != nullptr) {  // workgroup-uniform
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        const float rn = __builtin_amdgcn_rsqf(sum16(ss) * (1.f / D) + eps);
        const size_t tp = static_cast<size_t>(max(len(b) - 1, 0)) * (D / 2) + 8 * (l16 & 7);
        const float sg = l16 < 8 ? -1.f : 1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float z = x[e] * rn;
          x[e] = z;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float zp = dpp<0x128>(x[e]);  // row_ror:8, the partner lane's element
          qv[g][e] = fmaf(x[e], cos_t[tp + e], sg * sin_t[tp + e] * zp) * c2;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[g][e] = x[e] * c2;
      }
    }
  };
  float m[GQ], l[GQ], acc[GQ][8];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }
  auto compute = [&](const Batch& t, const uint4 (&xk)[U], const uint4 (&xv)[U]) {
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      float z[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        float a = 0.f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const uint32_t u = (&xk[i].x)[w4];
          a = fmaf(qv[g][2 * w4], __uint_as_float(u << 16), a);
          a = fmaf(qv[g][2 * w4 + 1], __uint_as_float(u & 0xffff0000u), a);
        }
        a = sum16(a);
        z[i] = t.j + i < t.jend ? a : -INFINITY;
      }
      // the batch's first row is always used, so m_new is finite
      float bm = z[0];
#pragma unroll
      for (int i = 1; i < U; ++i) bm = fmaxf(bm, z[i]);
      const float m_new = fmaxf(m[g], bm);
      const float alpha = fast_exp2(m[g] - m_new);  // 0 on a segment's first batch
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const float p = fast_exp2(z[i] - m_new);  // 0 for unused rows
        l[g] += p;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const uint32_t u = (&xv[i].x)[w4];
          acc[g][2 * w4] = fmaf(p, __uint_as_float(u << 16), acc[g][2 * w4]);
          acc[g][2 * w4 + 1] = fmaf(p, __uint_as_float(u & 0xffff0000u), acc[g][2 * w4 + 1]);
        }
      }
      m[g] = m_new;
    }
    if (t.j + U >= t.jend) {  // last batch of the segment: partials out, reset
      const int j0 = first_key(len(t.b));
      const int x_end = pre[t.b] + t.jend - j0;  // flattened end of the segment
      const int k = w - owner(pre[t.b]);         // the segment's index in its sequence
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        const size_t sw = (static_cast<size_t>(t.b) * SC + k) * H + h0 + g;
        float* op = opart + sw * D + 8 * l16;
        *reinterpret_cast<float4*>(op) =
            make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
        *reinterpret_cast<float4*>(op + 4) =
            make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        if (l16 == 0) {
          ml[2 * sw] = m[g] * 0.6931471805599453f;  // back to natural-log units
          ml[2 * sw + 1] = l[g];
        }
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
      }
      // the range that holds the sequence's last key records its segment count
      if (x_end == pre[t.b + 1] && tid == 0) nseg[t.b] = k + 1;
    }
  };

  uint4 ak[U], av[U], bk[U], bv[U];
  QRows qa, qb;
  Batch cur = segment(x_lo);
  rows(cur, ak, av);
  set_q(qrow(cur), cur.b);
  while (true) {
    Batch nx = next(cur);
    const bool nq = nx.b >= 0 && nx.b != cur.b;
    if (nx.b >= 0) {
      rows(nx, bk, bv);
      if (nq) qb = qrow(nx);  // a new segment: its query
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, ak, av);
    __builtin_amdgcn_sched_barrier(0);
    if (nx.b < 0) break;
    if (nq) set_q(qb, nx.b);
    cur = nx;
    nx = next(cur);
    const bool nq2 = nx.b >= 0 && nx.b != cur.b;
    if (nx.b >= 0) {
      rows(nx, ak, av);
      if (nq2) qa = qrow(nx);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, bk, bv);
    __builtin_amdgcn_sched_barrier(0);
    if (nx.b < 0) break;
    if (nq2) set_q(qa, nx.b);
    cur = nx;
  }
}

__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ opart, const float* __restrict__ ml, const int* __restrict__ nseg,
    const int* __restrict__ seqlens, u16* __restrict__ o, float* __restrict__ lse, int H,
    int T_cap, int win, int app) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int SC = seg_cap(T_cap);
  const int d = threadIdx.x;  // elements d and d + 64
  const float* mlb = ml + 2 * (static_cast<size_t>(b) * SC * H + h);  // segment k at 2 k H
  const float* opb = opart + (static_cast<size_t>(b) * SC * H + h) * D + d;  // at k H D
  // the count, the length and the first G segments' partials are loaded
  // together (every slot lies inside the workspace; slots past the count hold
  // stale values and get weight 0), so the common case of at most G segments
  // costs one memory round trip
  constexpr int G = 16;
  const int G0 = min(G, SC);
  float mv[G], lv[G], ov[G], ov2[G];
  const int nsr = nseg[b];
  const int sl = seqlens[b];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int k = i < G0 ? i : 0;
    mv[i] = mlb[2 * k * H];
    lv[i] = mlb[2 * k * H + 1];
    ov[i] = opb[static_cast<size_t>(k) * H * D];
    ov2[i] = opb[static_cast<size_t>(k) * H * D + 64];
  }
  const int L = min(max(sl, 0), T_cap - app) + app;
  // a sequence with no visible key has no segments (and no count written)
  const int ns = L > 0 ? nsr : 0;
  float M = -INFINITY, den = 0.f, num = 0.f, num2 = 0.f;
  // one pass over the segments in groups of G with a running max M
  for (int k0 = 0; k0 < ns; k0 += G) {
    if (k0 > 0) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int k = k0 + i < ns ? k0 + i : k0;
        mv[i] = mlb[2 * k * H];
        lv[i] = mlb[2 * k * H + 1];
        ov[i] = opb[static_cast<size_t>(k) * H * D];
        ov2[i] = opb[static_cast<size_t>(k) * H * D + 64];
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (k0 + i >= ns) mv[i] = -INFINITY;
    float gm = mv[0];
#pragma unroll
    for (int i = 1; i < G; ++i) gm = fmaxf(gm, mv[i]);
    const float M_new = fmaxf(M, gm);  // finite: segment k0 < ns exists
    const float sc = expf(M - M_new);  // 0 on the first group
    den *= sc;
    num *= sc;
    num2 *= sc;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float wgt = expf(mv[i] - M_new);  // 0 for segments past ns
      den = fmaf(wgt, k0 + i < ns ? lv[i] : 0.f, den);
      num = fmaf(wgt, k0 + i < ns ? ov[i] : 0.f, num);
      num2 = fmaf(wgt, k0 + i < ns ? ov2[i] : 0.f, num2);
    }
    M = M_new;
  }
  (void)win;
  const float out = ns > 0 ? num / den : 0.f, out2 = ns > 0 ? num2 / den : 0.f;
  o[(static_cast<size_t>(b) * H + h) * D + d] = __builtin_bit_cast(u16, to_bf16(out));
  o[(static_cast<size_t>(b) * H + h) * D + d + 64] = __builtin_bit_cast(u16, to_bf16(out2));
  if (lse != nullptr && d == 0)
    lse[static_cast<size_t>(b) * H + h] = ns > 0 ? M + logf(den) : -INFINITY;
}

}  // namespace

// Scratch for callers that cannot allocate (na_attn_decode_noalloc): a fixed
// array in every device's global memory, which holds the split-KV partials in
// place of a caller workspace.  Host code never uses the array's name as an
// address (on the host it is a stand-in, not a device pointer): the device
// address comes from hipGetSymbolAddress, looked up once per device with that
// device current and cached.  Every call on a device shares its array, so
// calls that overlap on one device race; nothing needs clearing between calls
// (the combine reads only the partials the split kernel of the same call
// wrote).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* cached[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    cached[dev] = p;
  }
  *ptr = cached[dev];
  return hipSuccess;
}

std::size_t decode_workspace_bytes(int B, int H, int T_cap) {
  const std::size_t bs = static_cast<std::size_t>(std::min(B, batch_cap(T_cap)));
  const std::size_t segs = bs * seg_cap(T_cap) * H;
  return segs * (D + 2) * sizeof(float) + bs * sizeof(int);
}

hipError_t launch_decode_bf16(const void* q, const void* kc, const void* vc, const int* seqlens,
                              void* o, float* lse, int B, int H, int Hk, int T_cap,
                              int window, void* ws, hipStream_t s, hipEvent_t const* ev,
                              const void* k_new, const void* v_new, const float* cos_t,
                              const float* sin_t, float eps, const void* ve, const void* gate) {
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  // a window that covers the whole cache is no window
  const int win = window >= 0 && window < T_cap - 1 ? window : -1;
  const int Bs = std::min(B, batch_cap(T_cap));  // sequences per split/combine pair
  const std::size_t segs = static_cast<std::size_t>(Bs) * seg_cap(T_cap) * H;
  float* opart = static_cast<float*>(ws);
  float* ml = opart + segs * D;
  int* nseg = reinterpret_cast<int*>(ml + 2 * segs);
  // persistent workgroups: a few per compute unit (the kernel uses fewer when
  // the sequences hold few keys)
  const int cus = device_cus();
  // grouped query heads: one 16-lane group per key/value head serves its 2 or
  // 4 query heads (each cached row loaded once); other ratios use one group
  // per query head
  const int G = H / Hk;
  const int gq = G == 2 || G == 4 ? G : 1;
  const int per_cu = gq > 1 ? kWgPerCuGrouped : kWgPerCu;
  hipError_t e = mark(ev, 0, s);
  if (e != hipSuccess) return e;
  const int app = k_new != nullptr ? 1 : 0;
  if (app) {
    e = launch_kv_append_bf16(k_new, v_new, const_cast<void*>(kc), const_cast<void*>(vc),
                              seqlens, B, 1, Hk, T_cap, cos_t, sin_t, eps, ve, gate, s);
    if (e != hipSuccess) return e;
  }
  auto* split = gq == 4   ? decode_split_kernel<4>
                : gq == 2 ? decode_split_kernel<2>
                          : decode_split_kernel<1>;
  // up to Bs sequences per pair of launches, reusing the workspace in stream order
  for (int b0 = 0; b0 < B; b0 += Bs) {
    const int nb = std::min(Bs, B - b0);
    const std::size_t qo = static_cast<std::size_t>(b0) * H * D;        // q, o rows
    const std::size_t co = static_cast<std::size_t>(b0) * T_cap * Hk * D;  // cache rows
    const long keys = static_cast<long>(nb) * T_cap;  // visible keys at most
    const int P = static_cast<int>(std::max<long>(1, std::min<long>(
        static_cast<long>(per_cu) * cus, (keys + KMIN - 1) / KMIN)));
    e = launch(split, dim3(P), dim3(16 * (H / gq)), 0, s, static_cast<const u16*>(q) + qo,
               static_cast<const u16*>(kc) + co, static_cast<const u16*>(vc) + co, seqlens + b0,
               opart, ml, nseg, nb, H, Hk, T_cap, scale, win, app, cos_t, sin_t, eps);
    if (e != hipSuccess) return e;
    if (b0 + Bs >= B && (e = mark(ev, 1, s)) != hipSuccess) return e;
    e = launch(decode_combine_kernel, dim3(H, nb), dim3(64), 0, s,
               static_cast<const float*>(opart), static_cast<const float*>(ml),
               static_cast<const int*>(nseg), seqlens + b0, static_cast<u16*>(o) + qo,
               lse != nullptr ? lse + static_cast<std::size_t>(b0) * H : nullptr, H, T_cap, win,
               app);
    if (e != hipSuccess) return e;
  }
  return mark(ev, 2, s);
}

}  // namespace na
