// Internal launcher declarations shared by the C-ABI layer (api.cpp) and the
// kernel translation units.  Every launcher assumes its arguments were already
// validated by api.cpp (sizes >= 1, D == 128, aligned, non-aliased) and returns
// the HIP status of its launches.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <tuple>
#include <utility>

namespace na {

constexpr int kHeadDim = 128;

// Sliding windows: window < 0 (or one that covers every earlier key) is plain
// causal attention; window W >= 0 keeps keys i - W .. i for query i.
// Hk: key/value heads (H a multiple of Hk; query head h reads head h / (H / Hk)),
// Hk = H for plain multi-head attention.

// bf16 forward: o, lse from q, k, v.  With cos_t non-null, q holds the raw
// query heads, RMS-normalised (eps) and rotated at positions t by the fp32
// (>= T, D/2) cos/sin tables as the forward loads them; the rotated bf16 rows
// are written to q_rot (B, T, H, D).
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int T, int H, int Hk, int window, hipStream_t s,
                           const float* cos_t = nullptr, const float* sin_t = nullptr,
                           float eps = 0.f, void* q_rot = nullptr);

// bf16 prefill over a KV cache: k_new, v_new (B, T, Hk, D) appended at cache
// rows lens[b] .. lens[b] + T - 1 (lens clamped to [0, Tc - T] on the device),
// then the T queries attend bottom-right causally over rows 0 .. lens[b] + r.
// lse may be null.
// With cos_t non-null, q and k_new hold raw heads that are RMS-normalised (eps)
// and rotated by the fp32 (>= Tc, D/2) cos/sin tables at their cache positions
// on the way (k_new in the append, q as the forward loads it).  With ve
// non-null, v_new gets the value-embedding gate v + 3 sigmoid(gate) ve in the
// append (ve (B, T, Hk, D), gate (B, T, Hk), bf16).
hipError_t launch_prefill_bf16(const void* q, const void* k_new, const void* v_new, void* kc,
                               void* vc, const int* lens, void* o, float* lse, int B, int T,
                               int H, int Hk, int Tc, int window, hipStream_t s,
                               const float* cos_t = nullptr, const float* sin_t = nullptr,
                               float eps = 0.f, const void* ve = nullptr,
                               const void* gate = nullptr);

// bf16 backward: delta, then dk/dv, then dq.
// ws: optional dS workspace of bwd_workspace_bytes(B, T, H) bytes; with it dQ
// is a GEMM over the stored dS, without it the dQ pass recomputes S and dP
// (plain causal only: a window needs the workspace).
// With q_raw non-null (the workspace path only), q and k are the rotated heads
// of the QK-norm + rotary prologue, q_raw and k_raw its inputs, and dq, dk are
// written as the gradients of q_raw and k_raw (the prologue's backward in the
// dQ GEMM's and the dK/dV pass's epilogues; tables fp32 (>= T, D/2)).
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* delta, void* ws, int B, int T, int H, int Hk, int window,
                           hipStream_t s, hipEvent_t const* ev = nullptr,
                           const void* q_raw = nullptr, const void* k_raw = nullptr,
                           const float* cos_t = nullptr, const float* sin_t = nullptr,
                           float eps = 0.f, const void* ve = nullptr,
                           const void* gate = nullptr, void* dve = nullptr,
                           void* dgate = nullptr);
std::size_t bwd_workspace_bytes(int B, int T, int H);

// bf16 append of T new key/value rows per sequence at cache rows
// clamp(lens[b], 0, Tc - T) .. + T - 1, with the optional QK norm + rotary
// embedding of the key rows (cos_t non-null) and value-embedding gate (ve
// non-null) on the way.
hipError_t launch_kv_append_bf16(const void* k_new, const void* v_new, void* kc, void* vc,
                                 const int* lens, int B, int T, int Hk, int Tc,
                                 const float* cos_t, const float* sin_t, float eps,
                                 const void* ve, const void* gate, hipStream_t s);

// Decode workspace layout and size (bytes).
std::size_t decode_workspace_bytes(int B, int H, int T_cap);
// The library's own decode scratch (na_attn_decode_noalloc): kDecodeScratchBytes
// of device memory per device; decode_scratch returns the current device's
// address of it (looked up once per device).
constexpr std::size_t kDecodeScratchBytes = std::size_t(16) << 20;
hipError_t decode_scratch(void** ptr);
// With k_new non-null, the new token's key/value rows (B, Hk, D) are first
// appended at row clamp(seqlens[b], 0, T_cap - 1) (launch_kv_append_bf16 with
// T = 1, rotated / gated as given) and the sequence then includes it; with
// cos_t non-null the query rows are raw heads, normalised and rotated at the
// query's position.
hipError_t launch_decode_bf16(const void* q, const void* kc, const void* vc, const int* seqlens,
                              void* o, float* lse, int B, int H, int Hk, int T_cap, int window,
                              void* ws, hipStream_t s, hipEvent_t const* ev = nullptr,
                              const void* k_new = nullptr, const void* v_new = nullptr,
                              const float* cos_t = nullptr, const float* sin_t = nullptr,
                              float eps = 0.f, const void* ve = nullptr,
                              const void* gate = nullptr);

// bf16 QK normalisation + rotary embedding of q (B, T, H, D) and k (B, T, Hk, D)
// at positions t + clamp(off[b], 0, T_tab - T) (off may be null: positions t)
// of the fp32 (T_tab, D/2) cos/sin tables.  Forward: outq, outk = y(q), y(k)
// (dyq, dyk unused).  Backward: outq, outk = gradients of the inputs given
// dyq, dyk, the gradients of the outputs.  q == nullptr: the key rows only.
hipError_t launch_qk_norm_rope_bf16(const void* q, const void* k, const void* dyq,
                                    const void* dyk, void* outq, void* outk, const float* cos_t,
                                    const float* sin_t, const int* off, int B, int T, int H,
                                    int Hk, int T_tab, float eps, bool backward, hipStream_t s);

// bf16 value-embedding gate over (B, T, Hk, D) rows with gate logits g (B, T, Hk).
// Forward (a = v): out = v + 3 sigmoid(g) ve.  Backward (a = dv'):
// out = dve = 3 sigmoid(g) dv', dgate = 3 sigmoid(g) (1 - sigmoid(g)) <ve, dv'>.
hipError_t launch_value_gate_bf16(const void* a, const void* ve, const void* gate, void* out,
                                  void* dgate, int B, int T, int Hk, bool backward,
                                  hipStream_t s);

// Compute units of the current device (cached per device; 256 if the query
// fails).  Persistent grids size themselves from it.  Safe to call from several
// threads: each cache slot is an atomic, and two threads that race on a slot's
// first query store the same value.
inline int device_cus() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Grid of a persistent kernel: per_cu workgroups per compute unit, never more
// than there are items.
inline unsigned persistent_grid(long items, int per_cu) {
  const long slots = static_cast<long>(device_cus()) * per_cu;
  return static_cast<unsigned>(items < slots ? items : slots);
}

// Records ev[i] on s when timing events were supplied.
inline hipError_t mark(hipEvent_t const* ev, int i, hipStream_t s) {
  return ev ? hipEventRecord(ev[i], s) : hipSuccess;
}

// fp32 forward and backward.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int T, int H, hipStream_t s);
hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* delta, int B, int T, int H, hipStream_t s);

template <typename Tuple, std::size_t... I>
inline void fill_argv(Tuple& t, void** argv, std::index_sequence<I...>) {
  ((argv[I] = static_cast<void*>(&std::get<I>(t))), ...);
}

// Launch helper returning the launch status directly (hipGetLastError would
// also report stale errors left by unrelated earlier calls).
template <typename... Params, typename... Args>
inline hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, std::size_t shmem,
                         hipStream_t stream, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  std::tuple<Params...> packed(static_cast<Params>(args)...);
  void* argv[sizeof...(Params)];
  fill_argv(packed, argv, std::index_sequence_for<Params...>{});
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem, stream);
}

}  // namespace na
