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
//   split:   persistent workgroups (two per compute unit) walk the non-empty
//            (sequence b, 64-key chunk) slots, all heads per workgroup, one
//            16-lane group per head reading whole 256-byte head rows.  Each
//            group streams a chunk's keys in batches of 4 with an online
//            softmax in registers; the next batch's K and V loads (possibly
//            the next slot's, with its query) are in flight while the current
//            batch is computed.  Writes unnormalised o_c and (m_c, l_c) per
//            (b, chunk, h).  Balancing slots rather than launching one
//            workgroup per chunk matters: the ragged lengths otherwise leave
//            compute units idle (measured 48% -> 56% of HBM bandwidth).
//   combine: one 64-thread workgroup per (b, h) (two elements per thread), one
//            pass with a running max:
//            o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
// Rows t >= L (and, with a window, rows before j0) are never read.  With H_kv
// key/value heads the cache is (B, T_cap, H_kv, D) and query head h reads head
// h / (H / H_kv); with 2 or 4 query heads per key/value head one 16-lane group
// loads each row of its key/value head once and scores it against all of
// them (d20 with 5 key/value heads: 48.7 -> 42 us, with four workgroups per
// compute unit instead of two).
#include <algorithm>
#include <mutex>

#include "device_common.hpp"
#include "internal.hpp"

namespace na {
namespace {

constexpr int D = kHeadDim;
constexpr int CHUNK = 64;        // keys per work slot
constexpr int U = 4;            // keys per batch (per 16-lane group)
constexpr int kWgPerCu = 2;     // persistent workgroups per compute unit
constexpr int kWgPerCuGrouped = 4;  // the same with grouped query heads (smaller workgroups)
constexpr int kMaxFlatB = 8192;  // up to this many sequences the slot list is flattened

__host__ __device__ inline int n_chunks(int T_cap) { return (T_cap + CHUNK - 1) / CHUNK; }

// workspace: o_part [B][NC][H][D] fp32, then ml [B][NC][H][2] fp32 (m_c, l_c)
//
// Persistent split: a workgroup of 16 H threads (one 16-lane group per head,
// lane i of a group owns bytes 16 i .. 16 i + 15 of the 256-byte head row)
// walks work slots (b, chunk c) with c * CHUNK < L_b, slot w = blockIdx.x,
// + gridDim.x, ...  Slots are numbered over the flattened list of non-empty
// chunks (prefix sums of ceil(L_b / CHUNK) in LDS), so every workgroup gets
// the same number of slots give or take one.  A slot's keys stream in
// batches of U rows; the K, V (and, at a slot change, q) loads of the next
// batch, which may belong to the next slot, are issued before the current
// batch is computed, so HBM latency hides behind the previous batch's work
// across slot boundaries.  At the end of a slot each group writes its
// unnormalised partial output and (m, l).
struct Batch {
  int slot;  // flattened slot index, or -1 past the end
  int b, c;  // sequence and chunk
  int n;     // keys of the chunk below L (rows c * CHUNK .. c * CHUNK + n - 1)
  int ib;    // batch within the chunk
  int j0;    // first visible key of the sequence
};

// GQ: query heads per 16-lane group.  GQ = 1: one group per query head (any
// H / H_kv).  GQ = H / H_kv > 1: one group per key/value head, which loads
// each cached row once and scores it against all GQ query heads that read it.
template <int GQ>
__global__ __launch_bounds__(512) void decode_split_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kc, const u16* __restrict__ vc,
    const int* __restrict__ seqlens, float* __restrict__ opart, float* __restrict__ ml, int B,
    int H, int Hk, int T_cap, float scale, int win, int app, const float* __restrict__ cos_t,
    const float* __restrict__ sin_t, float eps) {
  __shared__ int pre[kMaxFlatB + 1];  // pre[b] = non-empty chunks of sequences < b
  const int tid = threadIdx.x;
  const int gi = tid >> 4;  // 16-lane group
  const int l16 = tid & 15;
  const int NC = n_chunks(T_cap);
  const int P = gridDim.x;
  const bool flat = B <= kMaxFlatB;
  // app = 1: the new token was just appended at row seqlens[b] (clamped to
  // T_cap - 1), which the sequence now includes
  auto len = [&](int b) { return min(max(seqlens[b], 0), T_cap - app) + app; };
  // first visible key of a sequence of length L (win < 0: no window)
  auto first_key = [&](int L) { return win < 0 ? 0 : max(0, L - 1 - win); };
  // chunks holding a visible key: first_key(L) / CHUNK .. (L - 1) / CHUNK
  auto n_vis = [&](int L) { return L > 0 ? (L - 1) / CHUNK - first_key(L) / CHUNK + 1 : 0; };
  int total;  // number of slots
  if (flat) {
    // prefix sums of chunk counts: serial over blocks of SW sequences, each
    // block summed by the first SW threads (SW: a power of two no larger
    // than the workgroup, which may have only 16 threads)
    const int SW = blockDim.x >= 64 ? 64 : blockDim.x >= 32 ? 32 : 16;
    if (tid < SW) {
      int run = 0;
      for (int b0 = 0; b0 < B; b0 += SW) {
        const int b = b0 + tid;
        const int c = b < B ? n_vis(len(b)) : 0;
        int x = c;  // inclusive scan over SW lanes
        for (int o = 1; o < SW; o <<= 1) {
          const int y = __shfl_up(x, o, SW);
          if (tid >= o) x += y;
        }
        if (b < B) pre[b + 1] = run + x;
        run += __shfl(x, SW - 1, SW);
      }
      if (tid == 0) pre[0] = 0;
    }
    __syncthreads();
    total = pre[B];
  } else {
    total = B * NC;  // raw (b, c) grid; empty slots are skipped below
  }

  // slot -> (b, c): binary search in pre (flat) or direct (raw)
  auto locate = [&](int slot, Batch& t) {
    if (flat) {
      int lo = 0, hi = B - 1;  // largest b with pre[b] <= slot
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= slot) lo = mid; else hi = mid - 1;
      }
      t.b = lo;
      t.c = first_key(len(lo)) / CHUNK + slot - pre[lo];
    } else {
      t.b = slot / NC;
      t.c = slot % NC;
    }
    const int L = len(t.b);
    t.j0 = first_key(L);
    // <= 0 only for raw slots past L or wholly before the window
    t.n = t.c < t.j0 / CHUNK ? 0 : min(CHUNK, L - t.c * CHUNK);
    // batches wholly before j0 are skipped
    t.ib = t.c == t.j0 / CHUNK ? (t.j0 - t.c * CHUNK) / U : 0;
  };
  auto first_from = [&](int slot) {  // first non-empty slot >= slot (stride P)
    Batch t{-1, 0, 0, 0, 0, 0};
    for (; slot < total; slot += P) {
      locate(slot, t);
      if (t.n > 0) {
        t.slot = slot;
        return t;
      }
    }
    t.slot = -1;
    return t;
  };
  auto next = [&](const Batch& t) {
    if ((t.ib + 1) * U < t.n) {
      Batch u = t;
      ++u.ib;
      return u;
    }
    return first_from(t.slot + P);
  };

  // the cache has Hk key/value heads; query head h reads head h / (H / Hk);
  // this group serves query heads h0 .. h0 + GQ - 1
  const int hk = GQ == 1 ? gi / (H / Hk) : gi;
  const int h0 = GQ == 1 ? gi : gi * GQ;
  const size_t rs = static_cast<size_t>(Hk) * D;
  const float c2 = scale * 1.4426950408889634f;  // scores in the exp2 domain
  auto rows = [&](const Batch& t, uint4 (&xk)[U], uint4 (&xv)[U]) {
    const size_t base = (static_cast<size_t>(t.b) * T_cap + t.c * CHUNK) * rs +
                        static_cast<size_t>(hk) * D + 8 * l16;
    const int rsi = Hk * D;
    const int r_lo = t.j0 - t.c * CHUNK;  // rows before it lie before the window
#pragma unroll
    for (int i = 0; i < U; ++i) {
      // rows past n or before the window: row n-1 / the first visible row is
      // read again instead (zero weight), so no row outside the window is read
      const int r = min(max(t.ib * U + i, r_lo), t.n - 1) * rsi;
      xk[i] = ld16(kc + base + r);
      xv[i] = ld16(vc + base + r);
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
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = (&r.x[g].x)[w];
        x[2 * w] = __uint_as_float(u << 16);
        x[2 * w + 1] = __uint_as_float(u & 0xffff0000u);
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
        for (int w = 0; w < 4; ++w) {
          const uint32_t u = (&xk[i].x)[w];
          a = fmaf(qv[g][2 * w], __uint_as_float(u << 16), a);
          a = fmaf(qv[g][2 * w + 1], __uint_as_float(u & 0xffff0000u), a);
        }
        a = sum16(a);
        const int row = t.ib * U + i;
        z[i] = row < t.n && t.c * CHUNK + row >= t.j0 ? a : -INFINITY;
      }
      float bm = z[0];
#pragma unroll
      for (int i = 1; i < U; ++i) bm = fmaxf(bm, z[i]);
      const float m_new = fmaxf(m[g], bm);
      // -inf only while every key so far lies before the window: exponents
      // are then taken against 0 so that they give 0, not NaN
      const float mref = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m[g] - mref);  // 0 on a chunk's first batch
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const float p = fast_exp2(z[i] - mref);  // 0 for dropped rows
        l[g] += p;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t u = (&xv[i].x)[w];
          acc[g][2 * w] = fmaf(p, __uint_as_float(u << 16), acc[g][2 * w]);
          acc[g][2 * w + 1] = fmaf(p, __uint_as_float(u & 0xffff0000u), acc[g][2 * w + 1]);
        }
      }
      m[g] = m_new;
    }
    if ((t.ib + 1) * U >= t.n) {  // last batch of the chunk: partials out, reset
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        const size_t slotw = (static_cast<size_t>(t.b) * NC + t.c) * H + h0 + g;
        float* op = opart + slotw * D + 8 * l16;
        *reinterpret_cast<float4*>(op) =
            make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
        *reinterpret_cast<float4*>(op + 4) =
            make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        if (l16 == 0) {
          ml[2 * slotw] = m[g] * 0.6931471805599453f;  // back to natural-log units
          ml[2 * slotw + 1] = l[g];
        }
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
      }
    }
  };

  uint4 ak[U], av[U], bk[U], bv[U];
  QRows qa, qb;
  Batch cur = first_from(static_cast<int>(blockIdx.x));
  if (cur.slot < 0) return;  // uniform: no work for this workgroup
  rows(cur, ak, av);
  set_q(qrow(cur), cur.b);
  while (true) {
    Batch nx = next(cur);
    if (nx.slot >= 0) {
      rows(nx, bk, bv);
      if (nx.slot != cur.slot) qb = qrow(nx);  // a new slot: its query
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, ak, av);
    __builtin_amdgcn_sched_barrier(0);
    if (nx.slot < 0) break;
    if (nx.slot != cur.slot) set_q(qb, nx.b);
    cur = nx;
    nx = next(cur);
    if (nx.slot >= 0) {
      rows(nx, ak, av);
      if (nx.slot != cur.slot) qa = qrow(nx);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, bk, bv);
    __builtin_amdgcn_sched_barrier(0);
    if (nx.slot < 0) break;
    if (nx.slot != cur.slot) set_q(qa, nx.b);
    cur = nx;
  }
}

__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ opart, const float* __restrict__ ml,
    const int* __restrict__ seqlens, u16* __restrict__ o, float* __restrict__ lse, int H,
    int T_cap, int NC, int win, int app) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(max(seqlens[b], 0), T_cap - app) + app;
  const int nc = (L + CHUNK - 1) / CHUNK;                         // chunks end here
  const int c_lo = win < 0 || L == 0 ? 0 : max(0, L - 1 - win) / CHUNK;  // and start here
  const int d = threadIdx.x;  // elements d and d + 64
  const float* mlb = ml + 2 * (static_cast<size_t>(b) * NC * H + h);  // chunk c at 2 c H
  const float* opb = opart + (static_cast<size_t>(b) * NC * H + h) * D + d;  // chunk c at c H D
  float num2 = 0.f;
  // one pass over the chunks in groups of 16 (all loads of a group issued
  // before they are used), with a running max M
  constexpr int G = 16;
  float M = -INFINITY, den = 0.f, num = 0.f;
  for (int c0 = c_lo; c0 < nc; c0 += G) {
    float mv[G], lv[G], ov[G], ov2[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const bool ok = c0 + i < nc;
      const int c = ok ? c0 + i : c0;
      mv[i] = ok ? mlb[2 * c * H] : -INFINITY;
      lv[i] = mlb[2 * c * H + 1];
      ov[i] = opb[static_cast<size_t>(c) * H * D];
      ov2[i] = opb[static_cast<size_t>(c) * H * D + 64];
    }
    float gm = mv[0];
#pragma unroll
    for (int i = 1; i < G; ++i) gm = fmaxf(gm, mv[i]);
    const float M_new = fmaxf(M, gm);  // finite: chunk c0 < nc exists
    const float sc = expf(M - M_new);  // 0 on the first group
    den *= sc;
    num *= sc;
    num2 *= sc;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float w = expf(mv[i] - M_new);  // 0 for chunks past nc
      den = fmaf(w, lv[i], den);
      num = fmaf(w, ov[i], num);
      num2 = fmaf(w, ov2[i], num2);
    }
    M = M_new;
  }
  const float out = nc > 0 ? num / den : 0.f, out2 = nc > 0 ? num2 / den : 0.f;
  o[(static_cast<size_t>(b) * H + h) * D + d] = __builtin_bit_cast(u16, to_bf16(out));
  o[(static_cast<size_t>(b) * H + h) * D + d + 64] = __builtin_bit_cast(u16, to_bf16(out2));
  if (lse != nullptr && d == 0)
    lse[static_cast<size_t>(b) * H + h] = nc > 0 ? M + logf(den) : -INFINITY;
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
  const std::size_t slots = static_cast<std::size_t>(B) * n_chunks(T_cap) * H;
  return slots * (D + 2) * sizeof(float);
}

hipError_t launch_decode_bf16(const void* q, const void* kc, const void* vc, const int* seqlens,
                              void* o, float* lse, int B, int H, int Hk, int T_cap,
                              int window, void* ws, hipStream_t s, hipEvent_t const* ev,
                              const void* k_new, const void* v_new, const float* cos_t,
                              const float* sin_t, float eps, const void* ve, const void* gate) {
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const int NC = n_chunks(T_cap);
  // a window that covers the whole cache is no window
  const int win = window >= 0 && window < T_cap - 1 ? window : -1;
  float* opart = static_cast<float*>(ws);
  float* ml = opart + static_cast<std::size_t>(B) * NC * H * D;
  // persistent workgroups: a few per compute unit, never more than slots
  const int cus = device_cus();
  // grouped query heads: one 16-lane group per key/value head serves its 2 or
  // 4 query heads (each cached row loaded once); other ratios use one group
  // per query head
  const int G = H / Hk;
  const int gq = G == 2 || G == 4 ? G : 1;
  const long slots = static_cast<long>(B) * NC;
  const int per_cu = gq > 1 ? kWgPerCuGrouped : kWgPerCu;
  const int P = static_cast<int>(std::min<long>(slots, static_cast<long>(per_cu) * cus));
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
  e = launch(split, dim3(P), dim3(16 * (H / gq)), 0, s, static_cast<const u16*>(q),
             static_cast<const u16*>(kc), static_cast<const u16*>(vc), seqlens, opart, ml, B, H,
             Hk, T_cap, scale, win, app, cos_t, sin_t, eps);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, 1, s)) != hipSuccess) return e;
  e = launch(decode_combine_kernel, dim3(H, B), dim3(64), 0, s, static_cast<const float*>(opart),
             static_cast<const float*>(ml), seqlens, static_cast<u16*>(o), lse, H, T_cap, NC,
             win, app);
  if (e != hipSuccess) return e;
  return mark(ev, 2, s);
}

}  // namespace na
