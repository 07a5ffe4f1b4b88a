// Device-side building blocks for the gfx950 attention kernels: bf16 vector
// types, MFMA wrappers, conversions and wavefront (64-lane) reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace na {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16) on one wavefront.
// Operand lanes: A row m and B column n live in lane (m or n) mod 32; each
// lane holds 8 consecutive-k values of its half (lanes 32..63 hold the other
// half of k).  Result: lane l, element r holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even fp32 -> bf16.
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

__device__ __forceinline__ float bf16_to_f32(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Pack two fp32 values into one dword of two bf16 (lo first), round to
// nearest even: a single v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Sum over all 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// DPP lane permutation of x within each 16-lane row (no LDS traffic).
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}

// Sum over aligned groups of 16 lanes (one DPP row); every lane gets the sum.
// Butterfly: swap neighbours, swap pairs (quad_perm), then mirror within each
// half row and within the row.
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// Sixteen-byte global/LDS load and store through a 4 x dword vector.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// ld16 for data read once: a non-temporal load
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
// st16 for data not read again soon: a non-temporal store
__device__ __forceinline__ void st16_nt(void* p, uint4 v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight bf16 values (16 bytes, element 2i in the low half of dword i) to fp32
// and back (round to nearest even).
__device__ __forceinline__ void unpack8(uint4 v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack8(const float (&y)[8]) {
  return make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                    pack_bf16x2(y[6], y[7]));
}

// The row of a 32-key (or 32-query) block that lane l (mod 32) loads as the
// A operand of the score MFMA, chosen so that accumulator element r of lane l
// ends up holding block row 8*(l/32) + (r%8) + 16*(r/8).  That makes each
// group of 8 accumulator elements a contiguous run of 8 rows, which is exactly
// one lane's share of a 16-row k-chunk of the following MFMA.  It swaps bits
// 2 and 3 of m.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Block row held by accumulator element r of lane l after a perm_row-loaded
// score MFMA.
__device__ __forceinline__ int acc_row(int lane, int r) {
  return 8 * (lane >> 5) + (r & 7) + 16 * (r >> 3);
}

// ---------------------------------------------------------------------------
// Direct HBM -> LDS copies (buffer_load ... lds).  A raw buffer resource covers
// [base, base + bytes); a load at a byte offset >= bytes returns zeros, which
// the kernels use to pad ragged tiles without branches.
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  // word1: base[47:32], stride 0; word3: dword data format, no swizzle
  return i32x4{static_cast<int>(static_cast<uint32_t>(a)), static_cast<int>(a >> 32),
               static_cast<int>(bytes), 0x00020000};
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// Lane i copies the 16 (dma16) or 4 (dma4) bytes at byte offset voff of the
// buffer into LDS at lds + 16 i (lds + 4 i).  lds must be wave-uniform.  The
// copy is asynchronous and tracked by vmcnt alone: the compiler does not know
// about it, so callers order it with wait_vmem() and a barrier.
// The resource must be wave-uniform; readfirstlane states that to the compiler
// (and is free when it already sits in scalar registers).
__device__ __forceinline__ i32x4 uniform_rsrc(i32x4 r) {
  return i32x4{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
               __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}

__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(uniform_rsrc(rsrc)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// dma16 for data read once: the non-temporal policy streams it past the caches.
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :
               : "v"(voff), "s"(uniform_rsrc(rsrc)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(uniform_rsrc(rsrc)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Waits until every vector memory operation of this wavefront has completed
// (DMA copies landed in LDS, global stores acknowledged).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Waits until every LDS read of this wavefront has returned its data.  Placed
// before each barrier after which a DMA copy may overwrite an LDS buffer that
// was read before it: the copies are asm the compiler does not see as LDS
// writes, so the read's completion is made explicit rather than left to the
// barrier's lowering; the "memory" clobber also keeps the compiler from
// moving any LDS access across it.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// ... all but the N most recently issued ones (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j receives element j % 4 of the 4-element (8-byte) rows supplied by
// lanes 4 e + j / 4, e = 0..3: when lane i supplies the address of
// M[R + i / 4][C + 4 (i % 4)] of a bf16 matrix M, lane j gets M[R + e][C + j].
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ uint2 ds_read_tr16_at(uint32_t lds) {
  return __builtin_bit_cast(
      uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>(lds)));
}

// Eight-byte LDS write at an LDS byte address.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_st8(uint32_t lds, uint32_t lo, uint32_t hi) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(lds) = u32x2{lo, hi};
}

// Sixteen-byte LDS read at an LDS byte address.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ uint4 lds_ld16(uint32_t lds) {
  const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lds);
  return __builtin_bit_cast(uint4, v);
}

// ---------------------------------------------------------------------------
// Swizzled 64 x 128 bf16 tiles in LDS (query tiles of the backward, key and
// value tiles of the forward), filled by dma16 from HBM.  A tile is 64
// unpadded rows of 256 bytes; the 16-byte chunk c of row r sits at chunk
// c ^ tile_swz(r).  tile_swz is a bijection of r mod 16, so the row reads of
// an MFMA operand (16 lanes: one chunk of 16 different rows) touch 16
// different chunks; and its top two bits differ between any four consecutive
// rows, so the transposing reads (32 lanes: 64 bytes of 4 consecutive rows)
// touch 16 different chunks too.  With gfx950's 64 four-byte LDS banks both
// are free of bank conflicts.
constexpr uint32_t kTileBytes = 64 * 128 * 2;

__device__ __forceinline__ uint32_t tile_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Per-lane byte offsets, within a tile, of this lane's operand reads.
struct TileOffsets {
  uint32_t nat[8];    // row read: row perm_row(l32), elements 16 kc + 8 half .. + 7
  uint32_t tr[4][2];  // transposed read, column block db: rows 4 sub .. 4 sub + 3
};

__device__ __forceinline__ TileOffsets tile_operand_offsets(int lane) {
  TileOffsets o;
  const int half = lane >> 5;
  const int pr = perm_row(lane & 31);
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) o.nat[kc] = pr * 256 + 16 * ((2 * kc + half) ^ tile_swz(pr));
  // Lane i of 16-lane group g supplies row 8 (g / 2) + 4 sub + i / 4 and the
  // columns 32 db + 16 (g % 2) + 4 (i % 4) .. + 3; it then holds column
  // 32 db + lane % 32 of rows 8 (lane / 32) + 4 sub + 0..3, i.e. half of the
  // 8 rows its MFMA operand needs (the other half comes from sub ^ 1).
  const int g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int r = 8 * (g >> 1) + 4 * sub + (i >> 2);
      const int col = 32 * db + 16 * (g & 1) + 4 * (i & 3);
      o.tr[db][sub] = r * 256 + 16 * ((col >> 3) ^ tile_swz(r)) + 2 * (col & 7);
    }
  return o;
}

// Per-lane LDS byte addresses of one tile's operand reads (tile address plus
// TileOffsets), formed once per tile and kept in registers; row blocks and
// buffer choices go into the reads' immediate offsets.
struct TileAddr {
  uint32_t nat[8];
  uint32_t tr[4][2];
};

__device__ __forceinline__ void nat_addr(uint32_t tile, const TileOffsets& o, uint32_t (&a)[8]) {
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    a[kc] = tile + o.nat[kc];
    asm volatile("" : "+v"(a[kc]));  // keep the sum; do not re-add at every read
  }
}

__device__ __forceinline__ void tr_addr(uint32_t tile, const TileOffsets& o,
                                        uint32_t (&a)[4][2]) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      a[db][sub] = tile + o.tr[db][sub];
      asm volatile("" : "+v"(a[db][sub]));
    }
}

// Transposed operand (8 consecutive rows of one column per lane): rows
// off / 256 + 8 (lane / 32) + 0..7, column 32 db + lane % 32 of the tile
// behind t = a.tr[db].
__device__ __forceinline__ bf16x8 tr_operand(const uint32_t (&t)[2], uint32_t off) {
  const uint2 lo = ds_read_tr16_at(t[0] + off);
  const uint2 hi = ds_read_tr16_at(t[1] + off);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Per-lane source offset of the tile copy: wavefront w of a workgroup of NW
// wavefronts moves rows 4 (w + NW m) .. + 3, m = 0 .. 16 / NW - 1, one 1-KB
// dma16 each (lane i: 16 bytes of row + i / 16 into physical chunk i % 16).
// rsb is the byte stride between rows in HBM.
__device__ __forceinline__ uint32_t tile_copy_offset(int wave, int lane, uint32_t rsb) {
  const int drow = 4 * wave + (lane >> 4);
  return drow * rsb + 16 * ((lane & 15) ^ tile_swz(drow));
}

// Copies this wavefront's share of a 64 x 128 tile: rows of the buffer
// resource (rows past its end arrive as zeros) into the tile at LDS address
// tile.  NW (4 or 8) wavefronts share the copy.
// NT: the rows are read once (non-temporal copies).
template <int NW = 4, bool NT = false>
__device__ __forceinline__ void copy_tile(i32x4 rsrc, uint32_t voff, uint32_t rsb, uint32_t tile,
                                          int wave) {
  static_assert(NW == 4 || NW == 8, "16 row groups split evenly");
#pragma unroll
  for (int m = 0; m < 16 / NW; ++m) {
    if constexpr (NT)
      dma16_nt(rsrc, voff + 4 * NW * m * rsb, tile + 1024 * (wave + NW * m));
    else
      dma16(rsrc, voff + 4 * NW * m * rsb, tile + 1024 * (wave + NW * m));
  }
}

// Workgroup order.  The hardware hands workgroup i to XCD i % 8, and each XCD
// has its own L2; the maps below make the workgroups of one XCD cover a few
// heads' tiles close together in time, so the rows that all tiles of a head
// share stay in that XCD's L2.  (Falls back to head-fastest order when the
// head count is not a multiple of 8.)
//
// xcd_tile_map_grouped maps workgroup index bid to a (batch*head, tile) pair:
// within each XCD the heads are taken in groups of up to G and a group's tiles
// are ordered tile-major (tile 0 of every head of the group, then tile 1,
// ...).  With tile 0 the heaviest, the hardware's in-order dispatch then
// starts the heaviest tiles of a group first across the XCD's compute units (a
// longest-first list schedule), so the last group ends without a long tail; a
// group's rows still fit the XCD's L2 and the shared last-level cache.
constexpr int kHeadGroup = 4;  // heads per group (measured best for the d12..d26 shapes)

// reverse_heads: an XCD takes its heads last-first (the tile order inside a
// group is kept), e.g. to read first what a preceding pass wrote last.
__device__ __forceinline__ void xcd_tile_map_grouped(int bid, int BH, int n_tiles, int G, int& bh,
                                                     int& t, bool reverse_heads = false) {
  constexpr int kXcds = 8;
  if (BH % kXcds != 0) {
    bh = bid % BH;
    t = bid / BH;
    return;
  }
  const int x = bid % kXcds, w = bid / kXcds;
  const int hpx = BH / kXcds;  // heads per XCD
  const int grp = w / (G * n_tiles);
  const int gsz = min(G, hpx - grp * G);
  const int i = w - grp * G * n_tiles;
  t = i / gsz;
  const int hl = grp * G + i % gsz;  // head of this XCD
  bh = x + kXcds * (reverse_heads ? hpx - 1 - hl : hl);
}

// Persistent grids: one workgroup per slot (compute units x workgroups per
// compute unit), each taking work items round by round until they run out.
// Round r of workgroup w takes the virtual block index 8 j + w mod 8, so the
// item stays on the XCD the hardware gives workgroup w (w mod 8) and
// xcd_tile_map_grouped's order applies; the XCD's local order (heaviest tile
// first within each group of heads) is dealt to its W = gridDim / 8
// workgroups boustrophedon, j = r W + (r odd ? W - 1 - l : l) with l = w / 8,
// so a workgroup that drew a heavy tile in one round draws a light one in the
// next.  Indices grow with r: the first one past the item count ends the walk.
// The hardware dispatcher, fed one workgroup per item, leaves a slot idle for
// microseconds after a short workgroup ends.
__device__ __forceinline__ int persistent_item(int r) {
  const int w = static_cast<int>(blockIdx.x), G = static_cast<int>(gridDim.x);
  if (G % 8 != 0) return w + r * G;
  const int W = G / 8, l = w / 8;
  const int j = r * W + ((r & 1) ? W - 1 - l : l);
  return 8 * j + (w & 7);
}

// ---------------------------------------------------------------------------
// Transposed LDS tile: 128 rows (head-dim index d) x 64 columns (keys or
// queries) of bf16, row stride 128 bytes, no padding.  The 16-byte column
// group cg (columns 8 cg .. 8 cg + 7) of row d is stored at physical group
// cg ^ tsw(d).  With gfx950's 64 four-byte LDS banks this makes both access
// patterns below conflict-free: the 16-lane groups of a ds_read_b128 that
// reads one column group of 16 consecutive rows, and the 32-lane groups of
// the ds_write_b64 stores of tstore_4x8.
__device__ __forceinline__ int tsw(int d) { return ((d >> 1) ^ (d >> 4)) & 7; }

// Element offset of column group cg of row d.
__device__ __forceinline__ int toff(int d, int cg) { return d * 64 + ((cg ^ tsw(d)) << 3); }

// Store a 4-column x 8-row block into a transposed tile.  x[i] holds 16 bytes
// (rows 8 lchunk .. 8 lchunk + 7) of column 4 lrow + i.  Odd-lchunk threads
// walk the 8 rows in pair-swapped order so that each 32-lane store group
// covers both row parities (and so all 64 banks).
__device__ __forceinline__ void tstore_4x8(u16* tile, const uint4 (&x)[4], int lrow, int lchunk) {
  const int p = lchunk & 1;
  const uint32_t sel = p ? 0x07060302u : 0x05040100u;  // high or low halves of two dwords
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    const int el = e ^ p;  // row within the 8-row chunk; el >> 1 == w
    const uint32_t lo_sel = (e & 1) ? (sel ^ 0x02020202u) : sel;
    const uint32_t a = __builtin_amdgcn_perm((&x[1].x)[w], (&x[0].x)[w], lo_sel);
    const uint32_t b = __builtin_amdgcn_perm((&x[3].x)[w], (&x[2].x)[w], lo_sel);
    const int d = 8 * lchunk + el;
    *reinterpret_cast<uint2*>(&tile[toff(d, lrow >> 1) + 4 * (lrow & 1)]) = make_uint2(a, b);
  }
}

// ---------------------------------------------------------------------------
// MFMAs written as inline assembly, so that each value sits in the register
// file its users need: score chains accumulate in VGPRs, where the softmax
// VALU work reads them, while long-lived accumulators (dK, dV, O) and
// resident operands (K, V, Q) stay in AGPRs.  (With the compiler's builtins
// the choice is one form for the whole kernel, and with more than 256
// registers per lane the scores then come out in AGPRs and are copied back.)
// The compiler neither knows these are MFMAs nor inserts their hazard wait
// states, so the wrappers and the code around them keep gfx950's rules for
// v_mfma_f32_32x32x16_bf16 (the same numbers the compiler inserts around its
// builtins): a VALU write of an operand needs 2 wait states before the MFMA
// reads it (the "s_nop 1" below; a copy the compiler might place right before
// the statement is such a write), a VALU read of the result needs 12 after the
// MFMA issues (callers read a chain only after at least one further MFMA has
// issued behind it, or behind an explicit s_nop), back-to-back MFMAs that
// accumulate into the same registers need none, and VALU code that reads
// AGPR accumulators first waits behind a drain (s_nop 15, s_nop 7).
//
// Score chain link: d (VGPR) += a (VGPR) * b (AGPR).
__device__ __forceinline__ void mfma_chain(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// First link of a score chain: d holds the chain's initial value (LDS reads,
// or a copy the compiler may have placed just before).
__device__ __forceinline__ void mfma_chain_first(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// dK/dV accumulation: acc (AGPR) += a (VGPR) * b (VGPR, written by VALU).
__device__ __forceinline__ void mfma_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// First link of a chain with a separate initial value: d (VGPR) = a * b + c,
// c left intact (a persistent offset vector); d must not overlap the inputs.
__device__ __forceinline__ void mfma_chain_init(f32x16& d, bf16x8 a, bf16x8 b, const f32x16& c) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3"
               : "=&v"(d)
               : "v"(a), "a"(b), "v"(c));
}
// Wait states between the last accumulation into eight AGPR accumulators and
// any read of them (VALU code reads them back through v_accvgpr_read).
__device__ __forceinline__ void mfma_drain(f32x16 (&x)[4], f32x16 (&y)[4]) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]));
  asm volatile("" : "+a"(y[0]), "+a"(y[1]), "+a"(y[2]), "+a"(y[3]));
}

}  // namespace na
