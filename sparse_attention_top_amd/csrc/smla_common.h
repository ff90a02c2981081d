// Device and host pieces shared by the forward (sparse_mla.hip) and the
// backward (sparse_mla_bwd.hip) of the sparse MLA library for MI355X /
// gfx950: constants, raw LDS / MFMA instruction wrappers, the top-k
// compaction, the bf16 tile gather and the per-tile fragment reads and
// MFMA loops. Device code sits in an anonymous namespace (each translation
// unit inlines its own copy); host helpers with state (the per-device scratch
// pool) are inline functions of smla_host, one instance per process.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "sparse_mla.h"

namespace {


constexpr int kD = SPARSE_MLA_HEAD_DIM;  // 512
constexpr int kRowBytes = kD * 2;        // one bf16 row = 1 KiB
constexpr int kRowStride = kRowBytes + 32;  // LDS row pitch: 32 B of padding keeps both the K and the transposing V fragment reads free of bank conflicts (measured fastest of the pitches and swizzles tried)
constexpr int kBK = 32;                  // valid slots per tile
constexpr int kListCap = 2048;           // raw top-k entries compacted per segment
constexpr int kNumXcd = 8;               // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr int kXcdChunk = 64;            // consecutive tokens kept on one XCD (shared window rows)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyTau = 8.0f;  // log2 headroom before the reference max must move

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(LDS_AS const void*)p; }

// Optimisation barrier on a per-tile base address: keeps loop strength
// reduction from hoisting one address register per unrolled offset (the
// constant offsets then fold into the LDS instructions' offset fields).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// LDS fragment reads issued as raw instructions. The compiler does not track
// them, so (a) it cannot assume they alias an in-flight LDS-DMA prefetch and
// stall on that, and (b) every consumer must first pass the registers through
// lds_wait<N>(), an explicit lgkmcnt wait taking them as in/out operands (no
// use can be scheduled above it). LDS operations complete in order, so
// waiting until at most N are outstanding -- N = the number of LDS reads
// issued after this one -- completes it; any other LDS operation issued in
// between only makes the wait stricter.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_b64(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_b64(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int N, typename T>
__device__ __forceinline__ void lds_wait(T& a, T& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N, typename T>
__device__ __forceinline__ void lds_wait4(T& a, T& b, T& c, T& d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N));
}
template <int N, typename T, typename U>
__device__ __forceinline__ void lds_wait6(T& a, T& b, U& c, U& d, U& e, U& f) {
  asm volatile("s_waitcnt lgkmcnt(%6)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f) : "n"(N));
}

// S-phase MFMAs with their accumulators pinned to VGPRs (the O accumulator
// fills the AGPRs). The first k-step takes an inline-zero C operand, so no
// VALU write precedes the chain; accumulation into the same registers is
// interlocked by the hardware. Before VALU code reads the result,
// mfma_vgpr_drain() pads the MFMA-write -> VALU-read distance with wait
// states (more than the longest 16x16x32 latency).
__device__ __forceinline__ void mfma_s_first(f32x4& c, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x4& c, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
template <int N>
__device__ __forceinline__ void mfma_vgpr_drain(f32x4 (&c)[2][N]) {
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < N; ++j) asm volatile("" : "+v"(c[i][j]));
}

template <int N>
__device__ __forceinline__ void mfma_vgpr_drain2(f32x4 (&c)[2][2][N]) {
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < N; ++j) asm volatile("" : "+v"(c[i][h][j]));
}

// P.V MFMA accumulating into AGPRs (the constraint keeps the 128-register O
// accumulator in the AGPR file). Accumulating into the same registers is
// interlocked by the hardware; VALU reads of the result must first pass
// mfma_agpr_drain().
__device__ __forceinline__ void mfma_acc(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_agpr_drain(f32x4 (&c)[32]) {
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 32; ++i) asm volatile("" : "+a"(c[i]));
}

template <int I>
struct Int {
  static constexpr int value = I;
};
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Int<B>{});
    static_for<B + 1, E>(f);
  }
}


__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most n of this wave's vector-memory operations are
// outstanding (n rounded down to an encodable step; waiting more is safe).
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if (n < 16) {  // exact below 16
    static_for<0, 16>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if (n == k) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(k) : "memory");
    });
    return;
  }
  if (n >= 48) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
  else if (n >= 32) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  else if (n >= 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if (n >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (n >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if (n >= 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The lane index, computed where it is used (an asm the compiler cannot fold
// into an earlier value): for code after a long loop, so that lane-derived
// values need not stay live across it.
__device__ __forceinline__ int fresh_lane_id() {
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  return ln;
}

__device__ __forceinline__ int lane_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Block index -> virtual index: blocks are dispatched round-robin over the
// XCDs, so give each XCD runs of kXcdChunk consecutive virtual indices (a run
// of consecutive tokens shares most of its sliding-window rows in that XCD's
// L2). A bijection on [0, nb).
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  constexpr int per = kNumXcd * kXcdChunk;
  const int full = (nb / per) * per;
  if (b >= full) return b;
  const int x = b % kNumXcd, p = b / kNumXcd;
  return ((p / kXcdChunk) * kNumXcd + x) * kXcdChunk + (p % kXcdChunk);
}

// The two halves of compact_segment: the loads of the segment's entries (one
// per thread per chunk), and the compaction proper. A caller may issue other
// loads in between: memory loads complete in issue order, so loads issued
// before the entries would hold the compaction up until they land.
template <int NW, int CAP>
struct SegmentRaw {
  static constexpr int CH = NW * 64;     // entries per chunk (one per thread)
  static constexpr int MAXC = CAP / CH;  // chunks per segment (len <= CAP)
  int raw[MAXC];
};
// The loads take no branch (positions past len read entry len - 1 and are
// dropped by compact_finish), so that no wait for them is forced at a join;
// trow must hold at least one entry.
template <int NW, int CAP>
__device__ __forceinline__ void compact_load(SegmentRaw<NW, CAP>& r, const int32_t* __restrict__ trow, int len, int lane,
                                             int w) {
#pragma unroll
  for (int c = 0; c < SegmentRaw<NW, CAP>::MAXC; ++c) {
    const int pos = c * SegmentRaw<NW, CAP>::CH + w * 64 + lane;
    r.raw[c] = trow[max(min(pos, len - 1), 0)];
  }
}
// int64 rows: an entry is valid iff 0 <= v < nkv in 64-bit arithmetic (nkv <=
// 2^31); a valid entry is narrowed to int32, anything else becomes -1, so a
// value such as 2^32 + r never wraps onto row r. The rest is the int32 form's.
template <int NW, int CAP>
__device__ __forceinline__ void compact_load(SegmentRaw<NW, CAP>& r, const int64_t* __restrict__ trow, int len, int lane,
                                             int w, uint32_t nkv) {
#pragma unroll
  for (int c = 0; c < SegmentRaw<NW, CAP>::MAXC; ++c) {
    const int pos = c * SegmentRaw<NW, CAP>::CH + w * 64 + lane;
    const int64_t v = trow[max(min(pos, len - 1), 0)];
    r.raw[c] = (uint64_t)v < (uint64_t)nkv ? (int32_t)v : -1;
  }
}
template <int NW, typename SM, int CAP>
__device__ __forceinline__ int compact_finish(const SegmentRaw<NW, CAP>& rr, int len, uint32_t nkv, SM& sm, int lane,
                                              int w) {
  constexpr int MAXC = SegmentRaw<NW, CAP>::MAXC;
  int raw[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) raw[c] = (c * SegmentRaw<NW, CAP>::CH + w * 64 + lane) < len ? rr.raw[c] : -1;
  uint64_t bal[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) bal[c] = __ballot((uint32_t)raw[c] < nkv);
  if constexpr (NW == 1) {
    int base = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if ((uint32_t)raw[c] < nkv) sm.list[base + lane_rank(bal[c])] = raw[c];
      base += __popcll(bal[c]);
    }
    return __builtin_amdgcn_readfirstlane(base);
  } else {
    if (lane == 0) {
#pragma unroll
      for (int c = 0; c < MAXC; ++c) sm.wcount(c, w) = __popcll(bal[c]);
    }
    lds_barrier();
    int base = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      int off = 0, tot = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const int ci = __builtin_amdgcn_readfirstlane(sm.wcount(c, i));
        off += (i < w) ? ci : 0;
        tot += ci;
      }
      if ((uint32_t)raw[c] < nkv) sm.list[base + off + lane_rank(bal[c])] = raw[c];
      base += tot;
    }
    lds_barrier();
    return __builtin_amdgcn_readfirstlane(base);
  }
}
// Compact the valid entries of trow[0, len) into sm.list (order kept), with
// one round of loads and two workgroup barriers. Returns the count (uniform
// across the workgroup). The per-wave counts live in the tile area, which
// holds no tile then; the closing barrier keeps them until every wave has
// read them.
template <int NW, typename SM, int CAP = kListCap>
__device__ __forceinline__ int compact_segment(const int32_t* __restrict__ trow, int len, uint32_t nkv, SM& sm, int lane,
                                               int w) {
  SegmentRaw<NW, CAP> r;
  compact_load(r, trow, len, lane, w);
  return compact_finish<NW>(r, len, nkv, sm, lane, w);
}
template <int NW, typename SM, int CAP = kListCap>
__device__ __forceinline__ int compact_segment(const int64_t* __restrict__ trow, int len, uint32_t nkv, SM& sm, int lane,
                                               int w) {
  SegmentRaw<NW, CAP> r;
  compact_load(r, trow, len, lane, w, nkv);
  return compact_finish<NW>(r, len, nkv, sm, lane, w);
}

__device__ __forceinline__ int tile_rows(int i, int n) { return min(kBK, n - i * kBK); }

// A pointer that is the same in every lane, kept in scalar registers (a
// vector copy would be spilled in the tile loop, and its reload would wait
// for every gather in flight: scratch loads share the gathers' counter).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// One zero row of the pool: rows past a tile's count are gathered from here,
// and padded rows of other staged operands too.
__device__ __attribute__((aligned(256))) const uint16_t kZeroRowBf16[kD] = {};

// Number of LDS-DMA loads wave w issues for tile i: every row of an existing
// tile is gathered (past the count from the zero row).
template <int NW>
__device__ __forceinline__ int tile_dma(int i, int n, int w) {
  (void)w;
  return tile_rows(i, n) > 0 ? kBK / NW : 0;
}

// The gather of one tile of BK rows into an LDS ring buffer: one LDS-DMA
// instruction per row (lane L moves bytes [16 L, 16 L + 16) of the 1 KiB
// row). Rows past the tile's count come from the zero row, so that stale LDS
// never meets a zero probability (0 * NaN) and the issue has no branch per row
// (lane r picks row r's source, pool row or zero row, once per tile). Wave w
// moves rows [w RPW, (w+1) RPW).
template <int NW, int BK = kBK>
struct TileIssue {
  static constexpr int RPW = BK / NW;
  const uint16_t* kv;  // pool, in scalar registers
  uint32_t dst0;       // LDS address of this wave's first row in the target buffer
  int my;              // lane L < RPW: list entry of row r0 + L, or -1 past the tile's count
  bool active;

  // Tile i of the n-entry LDS list `list`, into the ring buffer at LDS address buf.
  __device__ __forceinline__ void init(const int32_t* list, int i, int n, bool act, uint32_t buf, const uint16_t* kv_,
                                       int lane, int w) {
    kv = uniform_ptr(kv_);
    active = act;
    const int r0 = w * RPW;
    const int cnt = act ? min(BK, n - i * BK) : 0;
    dst0 = buf + r0 * kRowStride;
    int e = -1;
    if (act && lane < RPW && r0 + lane < cnt) e = list[i * BK + r0 + lane];
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(e));
    my = e;
  }
  // As init, with this lane's list entry list[i BK + r0 + lane] already read
  // (any value where that position is at or past the tile's count).
  __device__ __forceinline__ void init_with(int e_read, int i, int n, bool act, uint32_t buf, const uint16_t* kv_,
                                            int lane, int w) {
    kv = uniform_ptr(kv_);
    active = act;
    const int r0 = w * RPW;
    const int cnt = act ? min(BK, n - i * BK) : 0;
    dst0 = buf + r0 * kRowStride;
    my = (act && lane < RPW && r0 + lane < cnt) ? e_read : -1;
  }
  // Lane L < RPW forms the 64-bit source address of row r0 + L once (vector
  // ops); each row then costs two lane reads, the LDS base and the load.
  // The row source addresses in scalar registers (formed ahead of the loads
  // when the caller holds them across other work).
  struct Rows {
    uint64_t a[RPW];
  };
  __device__ __forceinline__ void rows(Rows& r) const {
    const uint16_t* src = my >= 0 ? kv + (size_t)(uint32_t)my * kD : kZeroRowBf16;
    const uint64_t a = (uint64_t)(uintptr_t)src;
    const uint32_t alo = (uint32_t)a, ahi = (uint32_t)(a >> 32);
    static_for<0, RPW>([&](auto rc) {
      constexpr int RR = decltype(rc)::value;
      const uint32_t rlo = (uint32_t)__builtin_amdgcn_readlane(alo, RR);
      const uint32_t rhi = (uint32_t)__builtin_amdgcn_readlane(ahi, RR);
      r.a[RR] = ((uint64_t)rhi << 32) | rlo;
    });
  }
  __device__ __forceinline__ void issue(const Rows& r, int lane) const {
    if (!active) return;
    static_for<0, RPW>([&](auto rc) {
      constexpr int RR = decltype(rc)::value;
      const uint16_t* rs = (const uint16_t*)(uintptr_t)r.a[RR];
      __builtin_amdgcn_global_load_lds(rs + 8 * lane, (LDS_AS void*)(uintptr_t)(dst0 + RR * kRowStride), 16, 0, 0);
    });
  }
  __device__ __forceinline__ void all(int lane) const {
    if (!active) return;
    Rows r;  // all lane reads first: no read-to-load wait per row
    rows(r);
    issue(r, lane);
  }
  // LDS-DMA instructions all() issues
  __device__ __forceinline__ int count() const { return active ? RPW : 0; }
};


// Max over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- 16-row tiles (one wave of up to 16 heads) ----
constexpr int kBK16 = 16;  // rows per 16-row tile

__device__ __forceinline__ void mfma16_acc(f32x4& c, const u32x2& a, const u32x2& b) {
  asm volatile("v_mfma_f32_16x16x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// O^T += V^T P^T for a 16-row tile: per d-tile one transposing read gives
// lane (g, li) V[4g .. 4g+3][16 dt + li], the A operand of the 16x16x16 MFMA.
__device__ __forceinline__ void tile_pv16(uint32_t vrow, const bf16x4& pk, f32x4 (&acc)[32]) {
  asm volatile("s_nop 4" ::: "memory");  // P written by VALU, read by MFMA below
  constexpr int VPF = 6;
  constexpr int VST = VPF + 1;
  const u32x2 pb = __builtin_bit_cast(u32x2, pk);
  u32x2 vf[VST];
  auto vread = [&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    vf[dt % VST] = ds_read_tr16_b64<32 * dt>(vrow);
  };
  static_for<0, VPF>([&](auto dc) { vread(dc); });
  static_for<0, 32>([&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    if constexpr (dt + VPF < 32) vread(Int<dt + VPF>{});
    constexpr int younger = 31 - dt < VPF ? 31 - dt : VPF;
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(vf[dt % VST]) : "n"(younger));
    mfma16_acc(acc[dt], vf[dt % VST], pb);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// ---- per-tile compute of one wave (16 heads x 32 slots) ----
// Lane (g, li) owns head li of the wave's 16; LDS addresses are those of the
// tile's buffer.

// K fragment (MFMA A operand of S^T = K Q^T): lane holds K[slot sh*16 + li][32k + 8g .. +8).
__device__ __forceinline__ uint32_t k_frag_addr(uint32_t tile, int g, int li) {
  return opaque(tile + li * kRowStride + 16 * g);
}
// V^T fragment (MFMA A operand of O^T += V^T P^T): two transposing reads give
// lane V[4g .. 4g+3 and 16+4g .. 16+4g+3][16 dt + li]; this lane addresses row
// 4g + li/4 (and that + 16), bytes 8 (li & 3) + 32 dt.
__device__ __forceinline__ uint32_t v_frag_addr(uint32_t tile, int g, int li) {
  return opaque(tile + (4 * g + (li >> 2)) * kRowStride + 8 * (li & 3));
}

// S^T = K Q^T: s[sh] holds S^T[slot sh*16 + 4g + i][head li]. K fragments are
// read KPF k-steps ahead; with CH = 2, even and odd k-steps accumulate into
// separate registers (four independent MFMA chains), summed at the end.
template <int KPF, int CH>
__device__ __forceinline__ void tile_s(uint32_t krow, const bf16x8 (&qf)[16], f32x4 (&s)[2]) {
  static_assert(CH == 1 || CH == 2, "one or two chains per half");
  constexpr int KST = KPF + 1;
  f32x4 sp[2][2][1];  // [k parity][half][1]
  u32x4 kf[KST][2];
  auto kread = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    kf[k % KST][0] = ds_read_b128<64 * k>(krow);
    kf[k % KST][1] = ds_read_b128<16 * kRowStride + 64 * k>(krow);
  };
  static_for<0, KPF>([&](auto kc) { kread(kc); });
  static_for<0, 16>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int c = CH == 2 ? (k & 1) : 0;
    if constexpr (k + KPF < 16) kread(Int<k + KPF>{});
    constexpr int younger = 2 * (15 - k < KPF ? 15 - k : KPF);
    lds_wait<younger>(kf[k % KST][0], kf[k % KST][1]);
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      if constexpr (k < CH) mfma_s_first(sp[c][sh][0], kf[k % KST][sh], __builtin_bit_cast(u32x4, qf[k]));
      else mfma_s(sp[c][sh][0], kf[k % KST][sh], __builtin_bit_cast(u32x4, qf[k]));
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  if constexpr (CH == 2) {
    mfma_vgpr_drain2<1>(sp);
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) s[sh] = sp[0][sh][0] + sp[1][sh][0];
  } else {
    f32x4 (&s0)[2][1] = sp[0];
    mfma_vgpr_drain<1>(s0);
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) s[sh] = sp[0][sh][0];
  }
}

// Online softmax of one tile in base 2 with a lazy reference max: slots >= cnt
// are masked; P is rounded to bf16 into pk, already in the B-operand layout of
// the P.V MFMA (the C layout of S^T). When the tile's max exceeds the
// reference by more than kLazyTau, the reference moves and what earlier tiles
// accumulated is rescaled.
__device__ __forceinline__ void tile_softmax(const f32x4 (&s)[2], int cnt, float scale_log2, int g, float& m_ref,
                                             float& l_part, f32x4 (&acc)[32], bf16x8& pk) {
  float x[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int sh = 0; sh < 2; ++sh)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = sh * 16 + 4 * g + i;
      const float xv = slot < cnt ? s[sh][i] * scale_log2 : -INFINITY;
      x[sh][i] = xv;
      mx = __builtin_fmaxf(mx, xv);
    }
  mx = row4_max(mx);
  if (__ballot(mx > m_ref + kLazyTau) != 0ull) {
    const float m_new = __builtin_fmaxf(m_ref, mx);
    if (__ballot(m_ref != -INFINITY) != 0ull) {
      // rescale what earlier tiles accumulated (lanes whose reference is
      // still -inf have nothing accumulated: alpha = 0 keeps it 0)
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_part *= alpha;
      // in place, one accumulator register at a time (the accumulators live
      // in AGPRs; a vector multiply would stage them all in VGPRs)
#pragma unroll
      for (int dt = 0; dt < 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float e = acc[dt][i];
          float tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(e), "=&v"(tmp)
                       : "v"(alpha));
          acc[dt][i] = e;
        }
    }
    m_ref = m_new;
  }
  const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
  float ls = 0.f;
#pragma unroll
  for (int sh = 0; sh < 2; ++sh)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = __builtin_amdgcn_exp2f(x[sh][i] - mu);
      ls += pv;
      pk[sh * 4 + i] = (__bf16)pv;
    }
  l_part += ls;
}

// O^T += V^T P^T over the 32 d-tiles, VPF d-tiles of V^T fragments in flight.
__device__ __forceinline__ void tile_pv(uint32_t vrow, const bf16x8& pk, f32x4 (&acc)[32]) {
  asm volatile("s_nop 4" ::: "memory");  // P written by VALU, read by MFMA below
  constexpr int VPF = 5;
  constexpr int VST = VPF + 1;
  u32x2 vf[VST][2];
  auto vread = [&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    vf[dt % VST][0] = ds_read_tr16_b64<32 * dt>(vrow);
    vf[dt % VST][1] = ds_read_tr16_b64<16 * kRowStride + 32 * dt>(vrow);
  };
  static_for<0, VPF>([&](auto dc) { vread(dc); });
  static_for<0, 32>([&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    if constexpr (dt + VPF < 32) vread(Int<dt + VPF>{});
    constexpr int younger = 2 * (31 - dt < VPF ? 31 - dt : VPF);
    lds_wait<younger>(vf[dt % VST][0], vf[dt % VST][1]);
    const bf16x8 a = __builtin_bit_cast(
        bf16x8, u32x4{vf[dt % VST][0][0], vf[dt % VST][0][1], vf[dt % VST][1][0], vf[dt % VST][1][1]});
    mfma_acc(acc[dt], a, pk);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Two OCP FP8 E4M3 codes (bytes 2 HI .. 2 HI + 1 of x) -> two bf16 (exact:
// every code is a bf16 value; the two NaN codes stay NaN). gfx950's packed
// scaled conversion with scale 1, issued as asm: the compiler's lowering of its
// builtin keeps only the first element of the pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16(uint32_t x) {
  uint32_t r;
  if constexpr (HI) asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(x));
  else asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(x));
  return r;
}
// Eight codes (little-endian bytes of v) -> eight bf16 in the same order.
__device__ __forceinline__ u32x4 fp8x8_to_bf16(const u32x2& v) {
  return u32x4{fp8x2_to_bf16<false>(v[0]), fp8x2_to_bf16<true>(v[0]), fp8x2_to_bf16<false>(v[1]),
               fp8x2_to_bf16<true>(v[1])};
}

// The conversions and MFMAs here are inline asm, so the compiler inserts none
// of the wait states between an asm VALU write of a VGPR and its reader (an
// MFMA source needs two on CDNA3/4; four are given). Taking the converted
// values as in/out operands pins the conversion above the nops and the reader
// below them.
__device__ __forceinline__ void valu_to_mfma(u32x4& a, u32x4& b) {
  asm volatile("s_nop 3" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void valu_to_mfma(u32x4& a) { asm volatile("s_nop 3" : "+v"(a)); }

// An OCP FP8 E4M3 pool -> bf16 copies of its code values, 16 codes per thread
// per step (exact: every code value is a bf16 value; the two NaN codes stay
// NaN). The dequant scale is not applied here: the kernels fold it into the
// logit scale and the output scale, as the fp8 kernels do.
__global__ __launch_bounds__(256) void smla_fp8_pool_decode_kernel(const uint8_t* __restrict__ codes,
                                                                   uint16_t* __restrict__ out, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const u32x4 c = __builtin_nontemporal_load((const u32x4*)codes + i);
    u32x4 lo = fp8x8_to_bf16(u32x2{c[0], c[1]});
    u32x4 hi = fp8x8_to_bf16(u32x2{c[2], c[3]});
    valu_to_mfma(lo, hi);  // the asm conversions' results are read by the stores below
    u32x4* d = (u32x4*)out + 2 * i;
    d[0] = lo;
    d[1] = hi;
  }
}

// int64 top-k rows -> int32: a valid index (0 <= v < num_kv) becomes its row
// number, anything else -1, so an index at or past 2^31 can never alias a row.
__global__ __launch_bounds__(256) void smla_idx64_kernel(const int64_t* __restrict__ in, int32_t* __restrict__ out,
                                                         int64_t n, int64_t num_kv) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const int64_t v = in[i];
    out[i] = (v >= 0 && v < num_kv) ? (int32_t)v : -1;
  }
}

// Max and sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace

namespace smla_host {

// Compute units of a device (cached; 0 if unknown).
inline int cu_count(int dev) {
  static int cache[64];
  if (dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    cache[dev] = n;
  }
  return cache[dev];
}

// Stream-ordered scratch (the forward's split path and int64 rows, the
// backward) comes from a pool of our own per device that keeps up to
// kPoolKeepBytes of freed memory between calls (so that repeated calls do not
// map their scratch anew); memory above that returns to the device at the next
// synchronisation.
constexpr uint64_t kPoolKeepBytes = (uint64_t)9 << 29;  // 4.5 GiB
inline hipMemPool_t scratch_pool(int dev) {
  static std::mutex mu;
  static hipMemPool_t pools[64];
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (pools[dev] == nullptr) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    uint64_t keep = kPoolKeepBytes;
    (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    pools[dev] = pool;
  }
  return pools[dev];
}

inline bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

inline int current_device(int* dev) {
  if (hipGetDevice(dev) != hipSuccess || *dev < 0) {
    (void)hipGetLastError();
    return SMLA_ERR_NO_DEVICE;
  }
  return SMLA_OK;
}

}  // namespace smla_host
