// Sparse MLA prefill forward (DeepSeek-V4) for MI355X / gfx950 (CDNA4).
//
// Operation: "[Triton/Gluon] [GFX950][DSV4] Sparse MLA training backward"
// (aiter PR #4766), section "Contract" -- per token t and head h, softmax of
// scale * q.k over the valid gathered rows of a shared bf16 pool (K == V),
// with an optional per-head sink logit in the denominator only; outputs bf16
// o and a sink-inclusive natural-log lse. The C ABI is in
// include/sparse_mla.h.
//
// Kernel structure (a workgroup works on one token and group of heads at a
// time: one such unit per workgroup, or, in the persistent 128-head kernel,
// units dealt to each workgroup in an XCD-aware order):
//   1. the token's top-k row is read and its valid slots (0 <= idx < num_kv,
//      one unsigned compare) are compacted into an LDS list -- invalid slots
//      are never dereferenced, so NaN/Inf in unused pool rows cannot reach
//      the output (the fix described on "[Triton/Gluon] [CI] [gfx942] Tuned
//      sparse MLA prefill for DSv4.1-Flash TP4; fix attn_sink in Triton
//      fallback" (aiter PR #6002), description);
//   2. tiles of 32 valid rows (16 at H <= 16) are gathered global->LDS with
//      the CDNA4 LDS-DMA load (one wave instruction moves one whole 1 KiB row),
//      into a ring of NBUF buffers, so that one gather serves every head of the
//      workgroup and both contractions;
//   3. S^T = K Q^T on bf16 MFMA (16x16x32, fp32 accumulate), K read from LDS;
//   4. online softmax in base 2 (scale * log2 e folded into one multiply),
//      with lazy rescaling: the reference max only moves when a tile's max
//      exceeds it by more than 2^8, which is exact because the final
//      normalisation uses the same reference;
//   5. O^T += V^T P^T on bf16 MFMA, V read from the same LDS tile with the
//      gfx950 transposing LDS load, P rounded to bf16 (at four waves each wave
//      accumulates its 128 columns of d for all of the workgroup's heads, 64
//      in the D-split kernel and 128 in the 128-head one, from the P tiles the
//      waves publish in LDS);
//   6. the sink is folded into the max and the denominator at the end, o is
//      rounded to bf16 and lse converted back to natural log.
//
// Invalid (tail) rows of a partial tile are gathered from a zero row and
// their logits forced to -inf, so stale LDS contents never reach the output.


#include <algorithm>
#include <atomic>
#include <type_traits>

#include "smla_common.h"

namespace {

using namespace smla_host;

struct Params {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* topk;
  const int64_t* topk64;  // int64 rows, read by the 16-row kernel itself (topk unused then), else null
  const float* sink;
  uint16_t* out;
  float* lse;
  int T;
  int H;
  uint32_t nkv;  // min(num_kv, 2^31): slot valid iff (uint32)idx < nkv
  int topk_n;
  int head_groups;
  float scale_log2;  // scale * log2(e) (times the pool's dequant scale for fp8 pools)
  float out_scale;   // the pool's dequant scale (1 for bf16), applied to o at the end
};

// Split over the top-k row (few tokens): split `sp` of a row covers raw
// positions [sp * split_len, (sp + 1) * split_len); its partial results go to
// part_ml (reference max in log2 units, row sum) and part_o (O not yet
// normalised), indexed ((t * head_groups + hg) * nsplit + sp) * 16 NW + head.
struct SplitArgs {
  int nsplit;
  int split_len;
  float* part_o;
  float* part_ml;
};

// LDS of one workgroup: the compacted top-k list and one byte area that holds,
// in turn, the per-wave counts of the compaction, the ring of NBUF gathered
// tiles (bf16 rows at pitch kRowStride, or 16 KiB fp8 slab tiles), and at the
// end the output staging (16 rows of pitch kRowStride per wave). With an fp8
// pool and eight waves (kConv), two bf16 tiles precede the ring: the waves
// dequantise each gathered tile once into one of them and compute from it.
// D-split P.V exchange (four waves, bf16 pool): each wave's P tile in its MFMA
// B-operand layout (16 bytes per lane), and per head a factor: the rescale of
// the tile (1 when the reference max stayed), at the end the output scale.
// Empty otherwise, so that the other variants keep their LDS size (the
// one-wave fp8 workgroup fits four per CU at exactly 40 KiB).
template <bool DS>
struct DsExchange {};
template <>
struct DsExchange<true> {
  uint8_t pbuf[4 * 64 * 16];
  float fac[16 * 4];
};

template <int NW, int NBUF, bool FP8>
struct Smem : DsExchange<!FP8 && NW == 4> {
  static constexpr bool kConv = FP8 && NW == 8;
  static constexpr int kBf16Tile = kBK * kRowStride;
  static constexpr int kTileBytes = FP8 ? kBK * kD : kBf16Tile;
  static constexpr int kRingOff = kConv ? 2 * kBf16Tile : 0;
  static constexpr int kRingEnd = kRingOff + NBUF * kTileBytes;
  static constexpr int kStageBytes = NW * 16 * kRowStride;
  static constexpr int kAreaBytes = kRingEnd > kStageBytes ? kRingEnd : kStageBytes;
  // list entries per compaction segment: 1024 in the four-wave bf16 workgroup
  // (four top-k values per thread instead of eight: fewer registers live in
  // the prologue, 11 -> 4 spilled, and 4 KiB less LDS), 2048 otherwise
  static constexpr int kCap = (!FP8 && NW == 4) ? 1024 : kListCap;
  uint8_t area[kAreaBytes];
  int32_t list[kCap];
  static constexpr bool kDs = !FP8 && NW == 4;
  // gather ring slot b
  __device__ __forceinline__ uint32_t tile(int b) { return lds_addr(area + kRingOff + b * kTileBytes); }
  // dequantised bf16 tile b (kConv only)
  __device__ __forceinline__ uint32_t ctile(int b) { return lds_addr(area + b * kBf16Tile); }
  // output staging base
  __device__ __forceinline__ uint32_t stage() { return lds_addr(area); }
  __device__ __forceinline__ int32_t& wcount(int c, int w) { return ((int32_t*)area)[c * NW + w]; }
};

// gfx950 transposing read of 8-bit elements: in each 16-lane group, lane li
// fetches 8 bytes at its address and receives byte (li % 8) of the fetches of
// lanes 2m + li / 8, m = 0..7 -- with lane 2m + h addressing columns 8h..8h+7 of
// row m, lane li gets column li of the group's 8 rows.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr8_b64(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
// A row of zero codes: lanes whose row is past a tile's count gather from it.
__device__ __attribute__((aligned(64))) const uint8_t kZeroRow8[kD] = {};

// The gather of one tile of an fp8 pool (512-byte rows). The tile's LDS
// layout is slab-major: block k (1 KiB) holds d = 32k .. 32k+31 of all 32 rows,
// as two 16-byte chunks per row with chunk j of row r at 16 (r + 32 j). One
// LDS-DMA instruction fills one block (lane L fetches row L % 32, chunk L / 32),
// so a tile takes 16 instructions; wave w fills blocks [w SPW, (w+1) SPW). Rows
// past the tile's count are gathered from kZeroRow8.
template <int NW>
struct TileIssue8 {
  static constexpr int SPW = 16 / NW;
  const uint8_t* src;  // this lane's bytes of its row in the wave's first slab
  uint32_t dst0;       // the wave's first slab in the target buffer
  bool act;

  // The list entry is read with a raw LDS read (see ds_read_b128): read by a
  // compiled load, the compiler may first wait for every gather in flight,
  // not knowing that none of them writes the list.
  __device__ __forceinline__ void init(const int32_t* list, int i, int n, bool act_, uint32_t buf, const uint8_t* kv,
                                       int lane, int w) {
    act = act_;
    const int k0 = w * SPW;
    dst0 = buf + (uint32_t)k0 * 1024;
    const int cnt = act ? tile_rows(i, n) : 0;
    const bool valid = act && (lane & 31) < cnt;
    uint32_t e = 0;
    if (valid) {
      // (the lane index recomputed: an address kept live from the start was spilled)
      asm volatile("ds_read_b32 %0, %1" : "=v"(e) : "v"(lds_addr(list + i * kBK + (fresh_lane_id() & 31))));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(e));
    const uint8_t* row = valid ? uniform_ptr(kv) + ((uint64_t)e << 9) : uniform_ptr(kZeroRow8);
    src = row + (32 * k0 + 16 * (lane >> 5));
  }
  template <int S>
  __device__ __forceinline__ void slab(int lane) const {
    (void)lane;
    if (!act) return;
    __builtin_amdgcn_global_load_lds(src + 32 * S, (LDS_AS void*)(uintptr_t)(dst0 + S * 1024), 16, 0, 0);
  }
  __device__ __forceinline__ void all(int lane) const {
    static_for<0, SPW>([&](auto sc) { slab<decltype(sc)::value>(lane); });
  }
};


// S^T = K Q^T from an fp8 tile: the K fragment of half sh and k-step k
// (lane: row 16 sh + li, d = 32k + 8g .. +8) is 8 bytes at kaddr + 1024 k + 256 sh,
// kaddr = tile + 16 (li + 32 (g / 2)) + 8 (g % 2); converted to bf16 before the MFMA.
template <int KPF>
__device__ __forceinline__ void tile_s8(uint32_t kaddr, const bf16x8 (&qf)[16], f32x4 (&s)[2]) {
  constexpr int KST = KPF + 1;
  f32x4 sp[2];
  u32x2 kf[KST][2];
  auto kread = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    kf[k % KST][0] = ds_read_b64<1024 * k>(kaddr);
    kf[k % KST][1] = ds_read_b64<1024 * k + 256>(kaddr);
  };
  static_for<0, KPF>([&](auto kc) { kread(kc); });
  static_for<0, 16>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k + KPF < 16) kread(Int<k + KPF>{});
    constexpr int younger = 2 * (15 - k < KPF ? 15 - k : KPF);
    lds_wait<younger>(kf[k % KST][0], kf[k % KST][1]);
    u32x4 a0 = fp8x8_to_bf16(kf[k % KST][0]);
    u32x4 a1 = fp8x8_to_bf16(kf[k % KST][1]);
    valu_to_mfma(a0, a1);
    if constexpr (k == 0) {
      mfma_s_first(sp[0], a0, __builtin_bit_cast(u32x4, qf[k]));
      mfma_s_first(sp[1], a1, __builtin_bit_cast(u32x4, qf[k]));
    } else {
      mfma_s(sp[0], a0, __builtin_bit_cast(u32x4, qf[k]));
      mfma_s(sp[1], a1, __builtin_bit_cast(u32x4, qf[k]));
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // MFMA write -> VALU read distance
#pragma unroll
  for (int sh = 0; sh < 2; ++sh) {
    asm volatile("" : "+v"(sp[sh]));
    s[sh] = sp[sh];
  }
}

// V^T fragment base of an fp8 tile. The P fragment (the B operand, built from
// the S^T accumulator layout) holds slots 4g .. 4g+3 then 16+4g .. 16+4g+3, so
// the lanes of group g fetch rows R(m) = 4g + m (m < 4) and 16 + 4g + m - 4
// (m >= 4), m = li / 2, bytes 8 (li % 2) of the d-tile's 16-column chunk; the
// transposing read then hands lane (g, li) those 8 slots at d = 16 dt + li.
__device__ __forceinline__ uint32_t v8_frag_addr(uint32_t tile, int g, int li) {
  const int m = li >> 1;
  const int row = 4 * g + m + (m >= 4 ? 12 : 0);
  return opaque(tile + 16 * row + 8 * (li & 1));
}

// O^T += V^T P^T from an fp8 tile: the V^T fragment of d-tile dt is one
// transposing 8-bit read at vaddr + 1024 (dt / 2) + 512 (dt % 2).
__device__ __forceinline__ void tile_pv8(uint32_t vaddr, const bf16x8& pk, f32x4 (&acc)[32]) {
  asm volatile("s_nop 4" ::: "memory");  // P written by VALU, read by MFMA below
  constexpr int VPF = 6;
  constexpr int VST = VPF + 1;
  u32x2 vf[VST];
  auto vread = [&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    vf[dt % VST] = ds_read_tr8_b64<1024 * (dt / 2) + 512 * (dt % 2)>(vaddr);
  };
  static_for<0, VPF>([&](auto dc) { vread(dc); });
  static_for<0, 32>([&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    if constexpr (dt + VPF < 32) vread(Int<dt + VPF>{});
    constexpr int younger = 31 - dt < VPF ? 31 - dt : VPF;
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(vf[dt % VST]) : "n"(younger));
    u32x4 a = fp8x8_to_bf16(vf[dt % VST]);
    valu_to_mfma(a);
    mfma_acc(acc[dt], __builtin_bit_cast(bf16x8, a), pk);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Dequantisation of wave w's slabs of an fp8 tile (slab-major at src) into a
// bf16 tile at dst (rows at pitch kRowStride): lane L converts the 16 codes of
// row L % 32, d = 32 k + 16 (L / 32) .. +16 of each slab k it gathered. The
// reads are raw LDS reads (see ds_read_b128); the store half waits for them.
template <int NW>
struct SlabCodes {
  static constexpr int SPW = 16 / NW;
  u32x4 v[SPW];
  __device__ __forceinline__ void load(uint32_t src, int lane, int w) {
    const uint32_t a = opaque(src + (uint32_t)(w * SPW * 1024 + 16 * lane));
    static_for<0, SPW>([&](auto sc) { v[decltype(sc)::value] = ds_read_b128<1024 * decltype(sc)::value>(a); });
  }
  __device__ __forceinline__ void store(uint32_t dst, int lane, int w) {
    static_for<0, SPW>([&](auto sc) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[decltype(sc)::value])); });
    const uint32_t out = dst + (uint32_t)(lane & 31) * kRowStride + 32 * (lane >> 5);
    static_for<0, SPW>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const int k = w * SPW + s;
      u32x4 lo = fp8x8_to_bf16(u32x2{v[s][0], v[s][1]});
      u32x4 hi = fp8x8_to_bf16(u32x2{v[s][2], v[s][3]});
      valu_to_mfma(lo, hi);  // the asm conversions' results are read by the stores below
      *(LDS_AS u32x4*)(uintptr_t)(out + 64 * k) = lo;
      *(LDS_AS u32x4*)(uintptr_t)(out + 64 * k + 16) = hi;
    });
  }
};

// Sink and normalisation of one head: o = acc * oscale, lse in natural log.
// With no mass on any valid slot, o = 0 and lse is the sink itself (or -inf).
struct HeadEnd {
  float oscale, lse;
};
__device__ __forceinline__ HeadEnd head_end(float l_part, float m_ref, float sink, bool has_sink, float sink_l2) {
  const float lsum = row4_sum(l_part);
  if (lsum == 0.f) return {0.f, has_sink ? sink : -INFINITY};
  const float mf = has_sink ? __builtin_fmaxf(m_ref, sink_l2) : m_ref;
  const float a = __builtin_amdgcn_exp2f(m_ref - mf);
  const float lf = lsum * a + (has_sink ? __builtin_amdgcn_exp2f(sink_l2 - mf) : 0.f);
  return {a / lf, (mf + __builtin_amdgcn_logf(lf)) * kLn2};
}

__device__ __forceinline__ void load_q(bf16x8 (&qf)[16], const Params& p, int t, int head, int g) {
  // Q^T fragments (MFMA B operand of S^T = K Q^T): lane holds q[t, head, 32k + 8g .. +8).
  // q is read once: non-temporal loads leave the caches to the pool rows the
  // gathers reuse (2% at H = 128, where q and o stream 1 KiB per head).
  if (head < p.H) {
    const bf16x8* src = (const bf16x8*)(p.q + ((size_t)t * p.H + head) * kD + 8 * g);
#pragma unroll
    for (int k = 0; k < 16; ++k) qf[k] = __builtin_nontemporal_load(src + 4 * k);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) qf[k] = bf16x8{};
  }
}

// As load_q with no branch: a head past H loads head H - 1 (its results are
// never stored), so no wait for q is forced where control flow joins. Cached
// loads: each instruction reads one half of sixteen 128-byte lines and the
// next k-step the other half, which a non-temporal load may already have
// evicted (the 128-head kernel fetched 0.06 GB more per launch at T = 8192
// with non-temporal loads, and took 1% longer).
__device__ __forceinline__ void load_q_any(bf16x8 (&qf)[16], const Params& p, int t, int head, int g) {
  const bf16x8* src = (const bf16x8*)(p.q + ((size_t)t * p.H + min(head, p.H - 1)) * kD + 8 * g);
#pragma unroll
  for (int k = 0; k < 16; ++k) qf[k] = src[4 * k];
}

// ---- D-split P.V (four waves, 64 heads, bf16 pool) ----
// The wave that owns 16 heads computes their S and softmax, then publishes P
// (its B-operand fragment) and the per-head rescale factor in LDS; after a
// barrier every wave accumulates O^T for all 64 heads over its own 128 columns
// of d. Each V^T fragment read then feeds four MFMAs (one per head group)
// instead of one, so a tile's P.V reads 12 KiB of LDS per wave instead of 32.

// Online softmax of one tile as in tile_softmax, but the rescale factor of
// what earlier tiles accumulated is returned (1 when the reference max stays)
// instead of being applied: the accumulators of these heads are spread over
// all waves.
__device__ __forceinline__ float tile_softmax_ds(const f32x4 (&s)[2], int cnt, float scale_log2, int g, float& m_ref,
                                                 float& l_part, bf16x8& pk) {
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
  float alpha = 1.f;
  if (__ballot(mx > m_ref + kLazyTau) != 0ull) {
    const float m_new = __builtin_fmaxf(m_ref, mx);
    // a head whose reference is still -inf has nothing accumulated (alpha 0 keeps it 0)
    if (__ballot(m_ref != -INFINITY) != 0ull) alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
    l_part *= alpha;
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
  return alpha;
}

// Scale accumulator group o (8 d-tiles of one head group) by f, in place in
// the AGPRs, one register at a time.
__device__ __forceinline__ void scale_acc8(f32x4 (&acc)[32], int o, float f) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float e = acc[8 * o + dt][i];
      float tmp;
      asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                   : "+a"(e), "=&v"(tmp)
                   : "v"(f));
      acc[8 * o + dt][i] = e;
    }
}

// Apply the four head groups' published factors (lane li reads the factors
// of heads li, 16 + li, 32 + li, 48 + li); a group whose factors are all 1 is
// skipped.
__device__ __forceinline__ void apply_factors(f32x4 (&acc)[32], uint32_t fac_addr) {
  u32x4 f = ds_read_b128<0>(fac_addr);
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f));
#pragma unroll
  for (int o = 0; o < 4; ++o) {
    const float fo = __uint_as_float(f[o]);
    if (__ballot(fo != 1.f) != 0ull) scale_acc8(acc, o, fo);
  }
}

// O^T[128 w + 16 dt .. +16][heads 16 o + li] += V^T P_o^T for the wave's eight
// d-tiles and the four published P fragments. vrow: v_frag_addr of the tile
// plus the wave's 256-byte column offset; pbase: this lane's 16 bytes of head
// group 0's fragment (group o at + 1024 o).
__device__ __forceinline__ void tile_pv_ds(uint32_t vrow, uint32_t pbase, f32x4 (&acc)[32]) {
  asm volatile("s_nop 4" ::: "memory");  // accumulators rescaled by VALU, read by the MFMAs below
  constexpr int VPF = 3;
  constexpr int VST = VPF + 1;
  u32x4 pf[4];
  u32x2 vf[VST][2];
  static_for<0, 4>([&](auto oc) {
    constexpr int o = decltype(oc)::value;
    pf[o] = ds_read_b128<1024 * o>(pbase);
  });
  auto vread = [&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    vf[dt % VST][0] = ds_read_tr16_b64<32 * dt>(vrow);
    vf[dt % VST][1] = ds_read_tr16_b64<16 * kRowStride + 32 * dt>(vrow);
  };
  static_for<0, VPF>([&](auto dc) { vread(dc); });
  static_for<0, 8>([&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    if constexpr (dt + VPF < 8) vread(Int<dt + VPF>{});
    constexpr int younger = 2 * (7 - dt < VPF ? 7 - dt : VPF);
    if constexpr (dt == 0) lds_wait6<younger>(vf[0][0], vf[0][1], pf[0], pf[1], pf[2], pf[3]);
    else lds_wait<younger>(vf[dt % VST][0], vf[dt % VST][1]);
    const bf16x8 a = __builtin_bit_cast(
        bf16x8, u32x4{vf[dt % VST][0][0], vf[dt % VST][0][1], vf[dt % VST][1][0], vf[dt % VST][1][1]});
#pragma unroll
    for (int o = 0; o < 4; ++o) mfma_acc(acc[8 * o + dt], a, __builtin_bit_cast(bf16x8, pf[o]));
    __builtin_amdgcn_sched_barrier(0);
  });
}

// ---------------------------------------------------------------------------
// One workgroup per (token, group of 16 NW heads). Iteration j computes tile j
// from ring buffer j % NBUF while tiles j+1 .. j+NBUF-1 land; the rows of tile
// j+NBUF-1 are issued in one burst before P.V(j).
template <int NW, int NBUF, bool SPLIT, bool FP8>
__device__ __forceinline__ void smla_fwd_body(const Params& p, const SplitArgs& sa) {
  static_assert(NBUF >= 2 && NBUF <= 8, "ring of 2 to 8 tiles");
  constexpr int AHEAD = NBUF - 1;  // tiles gathered ahead of the one being computed
  using SM = Smem<NW, NBUF, FP8>;
  __shared__ __attribute__((aligned(16))) SM sm;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // 16-lane group
  const int li = lane & 15;  // index within the group

  const int vb = SPLIT ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  const int sp = SPLIT ? vb % sa.nsplit : 0;
  const int v = SPLIT ? vb / sa.nsplit : vb;
  const int t = p.T - 1 - v / p.head_groups;  // latest (heaviest) tokens first
  const int hg = v % p.head_groups;
  const int head_base = (hg * NW + w) * 16;
  const int head = head_base + li;
  const int row_begin = SPLIT ? min(p.topk_n, sp * sa.split_len) : 0;
  const int row_end = SPLIT ? min(p.topk_n, row_begin + sa.split_len) : p.topk_n;

  // D-split P.V: acc[8 o + dt] holds O^T[128 w + 16 dt + 4 g .. +4][head 16 o + li] of the
  // workgroup's 64 heads; otherwise acc[dt] holds O^T[16 dt + 4 g .. +4][head].
  constexpr bool DS = SM::kDs && !SPLIT;
  uint32_t pb_rd = 0, pb_own = 0, fac_rd = 0, fac_own = 0;
  if constexpr (SM::kDs) {
    pb_rd = lds_addr(sm.pbuf) + 16 * lane;          // P fragments, head group 0 (+1024 o)
    pb_own = pb_rd + 1024 * w;                      // this wave's P fragment
    fac_rd = lds_addr(sm.fac) + 16 * li;            // factors of heads li, 16 + li, 32 + li, 48 + li
    fac_own = lds_addr(sm.fac) + 16 * li + 4 * w;   // this lane's head
  }

  f32x4 acc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_part = 0.f;
  bf16x8 qf[16];
  load_q(qf, p, t, head, g);  // first, so that its latency overlaps the top-k row's
  bf16x8 pk;

  const int32_t* trow = p.topk + (size_t)t * p.topk_n;
  for (int seg0 = row_begin; seg0 < row_end; seg0 += SM::kCap) {
    if (seg0 > row_begin && NW > 1) lds_barrier();  // previous segment's list and tiles fully consumed
    const int n = compact_segment<NW, SM, SM::kCap>(trow + seg0, min(SM::kCap, row_end - seg0), p.nkv, sm, lane, w);
    const int ntiles = (n + kBK - 1) / kBK;
    if (ntiles == 0) continue;

    using Issue = typename std::conditional<FP8, TileIssue8<NW>, TileIssue<NW>>::type;
    using Elem = typename std::conditional<FP8, uint8_t, uint16_t>::type;
    const Elem* kvp = (const Elem*)p.kv;
    if constexpr (SM::kConv) {
      // Tile j: gathered into ring slot j % NBUF (NBUF tiles ahead), each wave
      // dequantises its own slabs into bf16 tile j % 2 one iteration ahead,
      // and all waves compute from that.
      constexpr int SPW = TileIssue8<NW>::SPW;
#pragma unroll
      for (int i = 0; i < NBUF; ++i) {
        Issue is;
        is.init(sm.list, i, n, i < ntiles, sm.tile(i), kvp, lane, w);
        is.all(lane);
      }
      int after0 = 0;
#pragma unroll
      for (int i = 1; i < NBUF; ++i) after0 += i < ntiles ? SPW : 0;
      wait_vmcnt_le(after0);
      SlabCodes<NW> codes;
      codes.load(sm.tile(0), lane, w);
      codes.store(sm.ctile(0), lane, w);
      for (int j = 0; j < ntiles; ++j) {
        lds_barrier();  // tile j dequantised by every wave; bf16 tile (j + 1) % 2 no longer read
        Issue is;
        is.init(sm.list, j + NBUF, n, j + NBUF < ntiles, sm.tile(j % NBUF), kvp, lane, w);
        is.all(lane);
        const uint32_t tb = sm.ctile(j & 1);
        f32x4 s[2];
        tile_s<2, 2>(k_frag_addr(tb, g, li), qf, s);
        tile_softmax(s, tile_rows(j, n), p.scale_log2, g, m_ref, l_part, acc, pk);
        if (j + 1 < ntiles) {
          int after = 0;  // this wave's gather loads issued after tile j+1's
#pragma unroll
          for (int i = 2; i <= NBUF; ++i) after += j + i < ntiles ? SPW : 0;
          wait_vmcnt_le(after);
          codes.load(sm.tile((j + 1) % NBUF), lane, w);
          codes.store(sm.ctile((j + 1) & 1), lane, w);
        }
        tile_pv(v_frag_addr(tb, g, li), pk, acc);
      }
      continue;
    }
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
      Issue is;
      is.init(sm.list, i, n, i < ntiles, sm.tile(i), kvp, lane, w);
      is.all(lane);
    }

    for (int j = 0; j < ntiles; ++j) {
      int after = 0;  // this wave's gather loads issued after tile j's
#pragma unroll
      for (int i = 1; i < AHEAD; ++i)
        if (j + i < ntiles) after += FP8 ? TileIssue8<NW>::SPW : tile_dma<NW>(j + i, n, w);
      wait_vmcnt_le(after);
      if constexpr (NW > 1) lds_barrier();
      Issue is;
      is.init(sm.list, j + AHEAD, n, j + AHEAD < ntiles, sm.tile((j + AHEAD) % NBUF), kvp, lane, w);
      const uint32_t tb = sm.tile(j % NBUF);
      f32x4 s[2];
      if constexpr (DS) {
        // S and softmax of this wave's heads; P and the rescale factor go to
        // LDS (the previous tile's were consumed before the barrier above)
        tile_s<2, 2>(k_frag_addr(tb, g, li), qf, s);
        // The softmax, the P exchange and the gather issue run at raised wave
        // priority, so that they pass ahead of the other workgroup's MFMA-bound
        // wave on this SIMD and the workgroup reaches its barrier sooner (1-2%).
        asm volatile("s_setprio 2" ::: "memory");
        const float alpha = tile_softmax_ds(s, tile_rows(j, n), p.scale_log2, g, m_ref, l_part, pk);
        *(LDS_AS bf16x8*)(uintptr_t)(pb_own) = pk;
        if (g == 0) *(LDS_AS float*)(uintptr_t)(fac_own) = alpha;
        lds_barrier();  // every wave's P and factors visible
        is.all(lane);
        apply_factors(acc, fac_rd);
        asm volatile("s_setprio 0" ::: "memory");
        tile_pv_ds(v_frag_addr(tb, g, li) + 256 * w, pb_rd, acc);
        continue;
      }
      if constexpr (FP8) tile_s8<2>(opaque(tb + 16 * (li + 32 * (g >> 1)) + 8 * (g & 1)), qf, s);
      else tile_s<2, 2>(k_frag_addr(tb, g, li), qf, s);
      tile_softmax(s, tile_rows(j, n), p.scale_log2, g, m_ref, l_part, acc, pk);
      is.all(lane);
      if constexpr (FP8) tile_pv8(v8_frag_addr(tb, g, li), pk, acc);
      else tile_pv(v_frag_addr(tb, g, li), pk, acc);
    }
  }

  if constexpr (SPLIT) {
    // partial results of this split; the merge kernel folds the splits and the sink
    mfma_agpr_drain(acc);
    const float lsum = row4_sum(l_part);
    const size_t pi = ((size_t)v * sa.nsplit + sp) * (16 * NW) + w * 16 + li;
    if (g == 0) {
      sa.part_ml[2 * pi] = m_ref;
      sa.part_ml[2 * pi + 1] = lsum;
    }
    float* dst = sa.part_o + pi * kD + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *(f32x4*)(dst + 16 * dt) = acc[dt];
    return;
  }

  // ---- finalise: fold the sink, normalise, store ----
  // o goes through LDS (row pitch kRowStride) so that each global store
  // writes one whole 1 KiB row per instruction. The sink is read only here,
  // so that its load latency is not on the way to the first tile.
  // lane-derived values are recomputed here rather than kept live across the
  // tile loop (where they would take registers, or be spilled)
  const int lane_f = fresh_lane_id(), g_f = lane_f >> 4, li_f = lane_f & 15, head_f = head_base + li_f;
  const float sk = (p.sink != nullptr && head_f < p.H) ? p.sink[head_f] : -INFINITY;
  const bool has_sink = !(sk == -INFINITY);
  const float sink_l2 = sk * kLog2e;
  HeadEnd he = head_end(l_part, m_ref, sk, has_sink, sink_l2);
  he.oscale *= p.out_scale;  // 1, or the dequant scale of an fp8 pool (V == code * scale)
  if (g_f == 0 && head_f < p.H) p.lse[(size_t)t * p.H + head_f] = he.lse;
  if constexpr (NW > 1) lds_barrier();  // all waves are done with the tiles
  const uint32_t ob = sm.stage() + (uint32_t)w * 16 * kRowStride;
  mfma_agpr_drain(acc);
  if constexpr (DS) {
    // every wave scales its columns of all 64 heads by the owners' output scales
    if (g_f == 0) *(LDS_AS float*)(uintptr_t)(lds_addr(sm.fac) + 16 * li_f + 4 * w) = he.oscale;
    lds_barrier();
    u32x4 f = ds_read_b128<0>(lds_addr(sm.fac) + 16 * li_f);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f));
    const uint32_t st = sm.stage() + 256 * w + 8 * g_f;  // row 16 o + li, bytes 2 (128 w + 16 dt + 4 g)
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      const float fo = __uint_as_float(f[o]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = acc[8 * o + dt] * fo;
        const bf16x4 v4 = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *(LDS_AS bf16x4*)(uintptr_t)(st + (16 * o + li_f) * kRowStride + 32 * dt) = v4;
      }
    }
    lds_barrier();  // the rows of every head staged
  }
  if constexpr (!DS) {
    // lane (g, li) holds o[head li][16 dt + 4g .. +4): write it to LDS row li
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const f32x4 o = acc[dt] * he.oscale;
      const bf16x4 ob4 = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
      *(LDS_AS bf16x4*)(uintptr_t)(ob + li_f * kRowStride + 32 * dt + 8 * g_f) = ob4;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  // row r of this wave's 16: lane L stores bytes [16 L, 16 L + 16) (non-temporal, like the q loads)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int hr = head_base + r;
    const u32x4 val = *(LDS_AS const u32x4*)(uintptr_t)(ob + r * kRowStride + 16 * lane_f);
    if (hr < p.H) __builtin_nontemporal_store(val, (u32x4*)(p.out + ((size_t)t * p.H + hr) * kD + 8 * lane_f));
  }
}

template <int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void smla_fwd_kernel(const Params p) {
  smla_fwd_body<NW, NBUF, false, false>(p, SplitArgs{});
}

// One workgroup per (token, head group, split of the top-k row); writes partial results.
template <int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void smla_fwd_split_kernel(
    const Params p, const SplitArgs sa) {
  smla_fwd_body<NW, NBUF, true, false>(p, sa);
}

// The same two kernels for a pool of OCP FP8 E4M3 codes.
template <int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void smla_fwd_fp8_kernel(
    const Params p) {
  smla_fwd_body<NW, NBUF, false, true>(p, SplitArgs{});
}
template <int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void smla_fwd_fp8_split_kernel(
    const Params p, const SplitArgs sa) {
  smla_fwd_body<NW, NBUF, true, true>(p, sa);
}

// ---------------------------------------------------------------------------
// H > 64, bf16 pool, single pass: four-wave workgroups, one per CU (one wave
// per SIMD, up to 512 registers), each working on one (token, group of 128
// heads) unit at a time and walking its share of the units (Sched128).
//
// Each wave owns 32 heads for S (Q^T of 32 heads in 128 VGPRs), so one K
// fragment read from LDS feeds two MFMAs; P of every head goes through LDS and
// each wave accumulates O^T for its 128 columns of d over all 128 heads (256
// AGPRs), so one V^T fragment read feeds eight MFMAs. Each row is gathered once
// per token (not once per 64-head group).
//
// With one wave per SIMD nothing else hides a wave's own latencies, so each
// tile is software-pipelined by hand: phase X accumulates P.V(j) and runs the
// softmax of tile j+1 between its MFMAs (publishing P(j+1)); after one barrier,
// phase Y computes S(j+2) and issues the rows of tile j+3 between its MFMAs. A
// 16x16x32 MFMA keeps the matrix pipe busy for about 16 cycles, during which
// the wave can issue about two other instructions, so the softmax is kept to
// about 80 instructions per tile: the reference max moves (a cross-lane
// reduction and rescale factors published for all waves) only when a lane's
// tile max passes its threshold, which after the first tile is rare. Tiles are
// gathered three ahead into a ring of four (also the 128-row output staging).

// The O^T accumulators of this kernel are kept by hand in the AGPR file:
// acc(o, dt) (head block o, d-tile dt) is a[32 o + 4 dt .. +3]. With all 256
// AGPRs holding live accumulators, the register allocator has no free AGPR for
// the copies it makes at loop joins and spills; here the compiler allocates
// no AGPR of its own (the kernel's VGPR demand stays below 256, so nothing is
// spilled into AGPRs), and one empty asm claims the whole file so the kernel's
// register allocation covers it.
#include "smla_acc128.h"

__device__ __forceinline__ void acc128_claim_and_zero() {
  asm volatile(SMLA_AGPR_ZERO_ASM ::: SMLA_ALL_AGPRS);
}
// acc(R / 32, (R % 32) / 4) += A B
template <int R>
__device__ __forceinline__ void acc128_mfma(const bf16x8& a, const bf16x8& b, float d0, float d1) {
  static_assert(R % 4 == 0 && R < 256, "one tuple of the AGPR file");
  acc128_mfma_t<R / 4>(a, b, d0, d1);
}
template <int R>
__device__ __forceinline__ f32x4 acc128_read() {
  float x0, x1, x2, x3;
  acc128_read_t<R / 4>(x0, x1, x2, x3);
  return f32x4{x0, x1, x2, x3};
}
template <int R>
__device__ __forceinline__ void acc128_scale(float f) {
  acc128_scale_t<R / 4>(f);
}

constexpr int k128Ring = 4;  // ring of 32-row tiles
constexpr int k128Ahead = k128Ring - 1;
constexpr int k128Cap = 1024;  // top-k entries compacted per segment

struct Smem128 {
  uint8_t area[k128Ring * kBK * kRowStride];  // gather ring
  uint8_t pbuf[2][8 * 64 * 16];               // P fragments of tile j, by tile parity: [head block][lane][16 B]
  float fac[2][128];                          // rescale factors, [li * 8 + head block], written with a flag
  uint8_t flag[2][4];                         // per wave (byte w): its factors of this tile were written
  float osc[128];                             // output scale of each head, [li * 8 + head block]
  int32_t list[2][k128Cap];                   // compacted lists of this unit and the next (by unit parity)
  int32_t wcnt[16];                           // per-wave counts of the compaction
  __device__ __forceinline__ uint32_t tile(int b) { return lds_addr(area + b * kBK * kRowStride); }
};
static_assert(sizeof(Smem128) <= 160 * 1024, "one workgroup per CU");

// An empty asm that "redefines" its operands: code using them cannot move above it.
template <typename T>
__device__ __forceinline__ void pin1(T& v) {
  asm volatile("" : "+v"(v));
}
template <typename... T>
__device__ __forceinline__ void pin(T&... v) {
  (pin1(v), ...);
}
// Plain v_max_f32 (the fmaxf lowering first canonicalises both operands, two
// more instructions; a NaN logit reaches the output through exp2 either way).
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ uint32_t bf16pair(float a, float b) {
  const bf16x4 v = bf16x4{(__bf16)a, (__bf16)b, (__bf16)0.f, (__bf16)0.f};
  return __builtin_bit_cast(u32x2, v)[0];
}

// S MFMA with operands it does not read (ordering only).
__device__ __forceinline__ void mfma_s_dep(f32x4& c, const u32x4& a, const u32x4& b, float d0, float d1) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b), "v"(d0), "v"(d1));
}
__device__ __forceinline__ void mfma_s_first_dep(f32x4& c, const u32x4& a, const u32x4& b, float d0, float d1) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b), "v"(d0), "v"(d1));
}

// The gather of one tile for the 128-head workgroup: wave w moves rows
// [8 w, 8 w + 8), lane L < 8 forming row 8 w + L's source address (a pool row,
// or the zero row past the tile's count, or for a tile past the unit's last);
// one LDS-DMA load per row, issued without a branch.
struct Gather128 {
  uint32_t dst0;      // LDS address of this wave's first row
  uint32_t alo, ahi;  // lane L < 8: source address of row L
  template <int R>
  __device__ __forceinline__ void row(int lane) const {
    const uint32_t rlo = (uint32_t)__builtin_amdgcn_readlane(alo, R);
    const uint32_t rhi = (uint32_t)__builtin_amdgcn_readlane(ahi, R);
    const uint16_t* rs = (const uint16_t*)(uintptr_t)(((uint64_t)rhi << 32) | rlo);
    __builtin_amdgcn_global_load_lds(rs + 8 * lane, (LDS_AS void*)(uintptr_t)(dst0 + R * kRowStride), 16, 0, 0);
  }
  __device__ __forceinline__ void all(int lane) const {
    static_for<0, kBK / 4>([&](auto rc) { row<decltype(rc)::value>(lane); });
  }
};
// The list entry of this lane's row (every lane reads an in-bounds entry, so no
// branch merges the pending register); the raw read is completed by a later
// wait that takes it as an operand.
__device__ __forceinline__ int opaque_lane(int lane) {  // recomputed at each use, not held in a register
  asm volatile("" : "+v"(lane));
  return lane;
}
__device__ __forceinline__ uint32_t gather128_read(const int32_t* list, int i, int lane, int w) {
  const int pos = min(i * kBK + w * (kBK / 4) + (opaque_lane(lane) & 7), k128Cap - 1);
  uint32_t e;
  asm volatile("ds_read_b32 %0, %1" : "=v"(e) : "v"(lds_addr(list + pos)));
  return e;
}
__device__ __forceinline__ Gather128 gather128_make(uint32_t e, int i, int n, bool act, uint32_t buf,
                                                   const uint16_t* kv, int lane, int w) {
  Gather128 ga;
  const int r0 = w * (kBK / 4);
  const int cnt = act ? min(kBK, n - i * kBK) : 0;
  ga.dst0 = buf + r0 * kRowStride;
  const bool have = act && lane < kBK / 4 && r0 + lane < cnt;
  const uint16_t* src = have ? uniform_ptr(kv) + (size_t)e * kD : kZeroRowBf16;
  const uint64_t a = (uint64_t)(uintptr_t)src;
  ga.alo = (uint32_t)a;
  ga.ahi = (uint32_t)(a >> 32);
  return ga;
}
__device__ __forceinline__ Gather128 gather128(const int32_t* list, int i, int n, bool act, uint32_t buf,
                                               const uint16_t* kv, int lane, int w) {
  uint32_t e = gather128_read(list, i, lane, w);
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(e));
  return gather128_make(e, i, n, act, buf, kv, lane, w);
}

// Phase Y: S = K Q^T from the tile at krow, 16 k-steps of four MFMAs (four
// independent chains), the K fragments of k-step u + KPF read between the
// first MFMAs of step u, and the rows of the next gather between the later
// ones. s[sh][hb] = S^T[slot 16 sh + 4g + i][head 32 w + 16 hb + li].
constexpr int kYKPF = 2;
struct NoTail {
  __device__ __forceinline__ void operator()() {}
};
struct NoGather {  // a phase Y with no gather
  template <int R>
  __device__ __forceinline__ void row(int) const {}
};
// tail() runs after the last MFMA is issued (the next phase's first reads).
template <typename GA, typename Tail = NoTail>
__device__ __forceinline__ void phase_y128(uint32_t krow, const bf16x8 (&qf)[2][16], f32x4 (&s)[2][2], const GA& ga,
                                           int lane, Tail&& tail = NoTail{}) {
  constexpr int KST = kYKPF + 1;
  u32x4 kf[KST][2];
  auto kread = [&](auto kc, auto hc) {
    constexpr int k = decltype(kc)::value, h = decltype(hc)::value;
    kf[k % KST][h] = ds_read_b128<16 * kRowStride * h + 64 * k>(krow);
  };
  static_for<0, kYKPF>([&](auto kc) {
    kread(kc, Int<0>{});
    kread(kc, Int<1>{});
  });
  static_for<0, 16>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    // reads issued after K(u): K(u+1) .. K(u+KPF-1)
    constexpr int wc = 2 * ((kYKPF - 1) < (15 - u) ? (kYKPF - 1) : (15 - u));
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(kf[u % KST][0]), "+v"(kf[u % KST][1]) : "n"(wc));
    static_for<0, 4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int sh = i >> 1, hb = i & 1;
      const u32x4 qb = __builtin_bit_cast(u32x4, qf[hb][u]);
      if constexpr (u == 0) mfma_s_first(s[sh][hb], kf[0][sh], qb);
      else mfma_s(s[sh][hb], kf[u % KST][sh], qb);
      if constexpr (i < 2 && u + kYKPF < 16) kread(Int<u + kYKPF>{}, Int<i>{});
      if constexpr (i == 2 && u % 2 == 0) ga.template row<u / 2>(lane);
      if constexpr (u == 15 && i == 3) tail();
    });
    __builtin_amdgcn_sched_barrier(0);
  });
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // MFMA write -> VALU read distance
#pragma unroll
  for (int sh = 0; sh < 2; ++sh)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) asm volatile("" : "+v"(s[sh][hb]));
}

// Per-token softmax state of this lane's two heads (32 w + 16 hb + li).
// The reference max m_ref (log2 units) is not kept: it is -nmu, or -inf while
// thr is -inf (nothing seen yet).
struct Soft128 {
  float l_part[2];  // this lane's share of the row sum relative to m_ref
  float nmu[2];     // -m_ref (0 while m_ref is -inf)
  float thr[2];     // a raw S value above this moves the reference: (m_ref + tau) / c
  __device__ __forceinline__ float m_ref(int hb) const { return thr[hb] == -INFINITY ? -INFINITY : -nmu[hb]; }
};
// Softmax temporaries of one tile.
struct SoftT {
  float t[2][4];
  float mxr[2];
  uint32_t flag;
};
struct Deps {
  float d0, d1;
};

// The rare step: a lane's tile max passed its threshold somewhere in the wave.
// Every head takes its row max across the four lanes; where that passes the
// reference by more than kLazyTau the reference moves to it and what earlier
// tiles accumulated is rescaled (factor published for every wave; 1 elsewhere).
// Exact: the final normalisation uses the same reference.
__device__ __forceinline__ void soft128_move(SoftT& tt, Soft128& ss, float c, float inv_c, uint32_t facw) {
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float mx = row4_max(tt.mxr[hb]) * c;
    const float mr = ss.m_ref(hb);
    const float mn = mx > mr + kLazyTau ? mx : mr;
    // a head whose reference is still -inf has nothing accumulated: its factor stays 1
    const float alpha = (mn == mr || mr == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mr - mn);
    ss.l_part[hb] *= alpha;
    ss.nmu[hb] = mn == -INFINITY ? 0.f : -mn;
    ss.thr[hb] = (mn + kLazyTau) * inv_c;
    *(LDS_AS float*)(uintptr_t)(facw + 4 * hb) = alpha;  // the four lanes of a head write the same value
  }
  tt.flag = 1;
}

// Group G of the softmax of one tile, run between two MFMAs of phase X. The
// logits are scale * log2(e) * S with the scale taken positive (q is negated
// for a negative scale), so the max is taken on S itself and p = 2^(c S - m)
// is one fma and one exp2. MASK: the tile is partial (slots >= cnt -> -inf).
template <int G, bool MASK>
__device__ __forceinline__ Deps soft128_group(f32x4 (&s)[2][2], SoftT& tt, Soft128& ss, float c, float inv_c, int cnt,
                                              int g, uint32_t pbw, uint32_t facw, uint32_t flagw) {
  constexpr int M = MASK ? 8 : 0;
  if constexpr (MASK && G < 8) {  // two elements (hb = G & 1, e = 2 (G >> 1) ..) past the count -> -inf
    constexpr int hb = G & 1, e0 = 2 * (G >> 1), sh = e0 >> 2, i0 = e0 & 3;
    pin(s[sh][hb]);
    const int lim = cnt - 4 * g;  // slot 16 sh + 4 g + i is valid iff 16 sh + i < lim
#pragma unroll
    for (int i = i0; i < i0 + 2; ++i) s[sh][hb][i] = (16 * sh + i) < lim ? s[sh][hb][i] : -INFINITY;
    return {s[sh][hb][i0], s[sh][hb][i0 + 1]};
  } else if constexpr (G < M + 4) {  // tile max, in-lane: two three-way maxima per group
    constexpr int hb = (G - M) & 1, part = (G - M) >> 1;
    pin(s[0][hb], s[1][hb]);
    if constexpr (part == 0) {
      tt.t[hb][0] = vmax3(s[0][hb][0], s[0][hb][1], s[0][hb][2]);
      tt.t[hb][1] = vmax3(s[0][hb][3], s[1][hb][0], s[1][hb][1]);
      return {tt.t[hb][0], tt.t[hb][1]};
    } else {
      pin(tt.t[hb][0], tt.t[hb][1]);
      tt.t[hb][2] = vmax3(s[1][hb][2], s[1][hb][3], tt.t[hb][0]);
      tt.mxr[hb] = vmax(tt.t[hb][2], tt.t[hb][1]);
      return {tt.mxr[hb], tt.mxr[hb]};
    }
  } else if constexpr (G < M + 8) {  // (free slots)
    return {c, c};
  } else if constexpr (G == M + 8) {  // does the reference move (rare)?
    pin(tt.mxr[0], tt.mxr[1], ss.thr[0], ss.thr[1]);
    tt.flag = 0;
    if (__ballot(tt.mxr[0] > ss.thr[0] || tt.mxr[1] > ss.thr[1]) != 0ull) soft128_move(tt, ss, c, inv_c, facw);
    return {ss.nmu[0], ss.nmu[1]};
  } else if constexpr (G < M + 25) {  // p = 2^(c S - m), in place
    constexpr int k = G - M - 9, hb = k & 1, e = k >> 1, sh = e >> 2, i = e & 3;
    pin(s[sh][hb], ss.nmu[hb]);
    s[sh][hb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sh][hb][i], c, ss.nmu[hb]));
    return {s[sh][hb][i], s[sh][hb][i]};
  } else if constexpr (G < M + 29) {  // P in bf16 (the B-operand layout of the P.V MFMA), published
    constexpr int hb = (G - M - 25) & 1, sh = (G - M - 25) >> 1;
    pin(s[sh][hb]);
    const u32x2 pk = u32x2{bf16pair(s[sh][hb][0], s[sh][hb][1]), bf16pair(s[sh][hb][2], s[sh][hb][3])};
    *(LDS_AS u32x2*)(uintptr_t)(pbw + 1024 * hb + 8 * sh) = pk;
    return {__uint_as_float(pk[0]), __uint_as_float(pk[1])};
  } else if constexpr (G < M + 33) {  // row sums of the fp32 p, in place: pairs
    constexpr int hb = (G - M - 29) & 1, sh = (G - M - 29) >> 1;
    pin(s[sh][hb]);
    s[sh][hb][0] = s[sh][hb][0] + s[sh][hb][1];
    s[sh][hb][2] = s[sh][hb][2] + s[sh][hb][3];
    return {s[sh][hb][0], s[sh][hb][2]};
  } else if constexpr (G < M + 35) {
    constexpr int hb = (G - M - 33) & 1;
    pin(s[0][hb], s[1][hb]);
    s[0][hb][0] = s[0][hb][0] + s[0][hb][2];
    s[1][hb][0] = s[1][hb][0] + s[1][hb][2];
    return {s[0][hb][0], s[1][hb][0]};
  } else if constexpr (G < M + 37) {
    constexpr int hb = (G - M - 35) & 1;
    pin(s[0][hb], s[1][hb], ss.l_part[hb]);
    ss.l_part[hb] += s[0][hb][0] + s[1][hb][0];
    return {ss.l_part[hb], ss.l_part[hb]};
  } else if constexpr (G == M + 37) {  // publish whether factors were written
    pin(tt.flag);
    *(LDS_AS uint8_t*)(uintptr_t)(flagw) = (uint8_t)tt.flag;
    return {c, c};
  } else {
    return {c, c};
  }
}
template <bool MASK>
constexpr int kSoftGroups128 = MASK ? 46 : 38;

// The whole softmax of one tile with no MFMAs to interleave (the first tile).
template <bool MASK>
__device__ __forceinline__ void soft128_plain(f32x4 (&s)[2][2], Soft128& ss, float c, float inv_c, int cnt, int g,
                                              uint32_t pbw, uint32_t facw, uint32_t flagw) {
  SoftT tt;
  static_for<0, kSoftGroups128<MASK>>([&](auto gc) {
    (void)soft128_group<decltype(gc)::value, MASK>(s, tt, ss, c, inv_c, cnt, g, pbw, facw, flagw);
  });
}

// The first LDS reads of phase X, issued ahead (during the previous phase Y,
// or right after the barrier): the list entry of the gather after next, the
// four wave flags (one dword), the P fragments of head blocks 0..3 and the
// first kXVPF V fragments. Completed by the waits of phase X, which take them
// as operands.
constexpr int kXVPF = 2;
struct XPre {
  uint32_t e;
  uint32_t fl;  // byte w: wave w's flag
  u32x4 pf[4];
  u32x2 vf[kXVPF + 1][2];  // the V^T fragment ring of phase X; the first VPF prefetched
};
__device__ __forceinline__ void x_prefetch(XPre& xp, const int32_t* list, int gi, int lane, int w, uint32_t flag_rd,
                                           uint32_t pbase, uint32_t vrow) {
  xp.e = gather128_read(list, gi, lane, w);
  asm volatile("ds_read_b32 %0, %1" : "=v"(xp.fl) : "v"(flag_rd));
  static_for<0, 4>([&](auto oc) { xp.pf[decltype(oc)::value] = ds_read_b128<1024 * decltype(oc)::value>(pbase); });
  static_for<0, kXVPF>([&](auto pc) {
    constexpr int pp = decltype(pc)::value;
    xp.vf[pp][0] = ds_read_tr16_b64<32 * pp>(vrow);
    xp.vf[pp][1] = ds_read_tr16_b64<16 * kRowStride + 32 * pp>(vrow);
  });
}

// Phase X LDS reads, in issue order: the prefetch above (1 + 1 + 4 + 2 VPF
// reads); at step u, V(u + VPF) between its first two MFMAs; at step 7 the P
// fragments of head blocks 4..7, each into the register of the one its MFMA
// has just read. Step u multiplies d-tile u % 8 with head blocks 4 (u / 8) .. +4
// (V(u): the V^T fragment of that d-tile; each is read twice). The factors,
// when a flag is set, are read and waited for apart.
struct PhaseX128 {
  static constexpr int kPro = 2 + 4 + 2 * kXVPF;
  static constexpr int before(int u) {  // reads issued before the wait of step u
    int r = kPro;
    for (int s = 0; s < u; ++s) r += (s + kXVPF < 16 ? 2 : 0) + (s == 7 ? 4 : 0);
    return r;
  }
  static constexpr int pos_v(int p) {
    if (p < kXVPF) return 6 + 2 * (p + 1);
    const int s = p - kXVPF;  // issued in step s: V half 0, [P 4], V half 1 at step 7
    return before(s) + (s == 7 ? 3 : 2);
  }
  static constexpr int wait_at(int u) {
    int need = pos_v(u);
    if (u == 0 && need < 6) need = 6;
    if (u == 8 && need < before(8)) need = before(8);  // the P fragments of head blocks 4..7
    return before(u) - need;
  }
};

// Slot k (MFMA k of 64) of phase X runs softmax group (k NG) / 64 when that is
// the first slot of its group: NG groups spread evenly over the 64 MFMAs.
template <int NG>
constexpr int soft_group_at(int k) {
  return (k * NG) % 64 < NG ? (k * NG) / 64 : -1;
}

// Phase X of iteration j: apply the factors of tile j (if a wave moved its
// references), then O^T += V^T P^T for the wave's 8 d-tiles x 8 head blocks,
// with the softmax groups of tile j+1 between the MFMAs (SOFT; MASK: tile j+1
// is partial). xp: the prefetched reads, completed here.
template <bool SOFT, bool MASK>
__device__ __forceinline__ void phase_x128(XPre& xp, uint32_t vrow, uint32_t pbase, uint32_t fac_rd, f32x4 (&s)[2][2],
                                           Soft128& ss, float c, float inv_c, int cnt, int g, uint32_t pbw,
                                           uint32_t facw, uint32_t flagw) {
  using Px = PhaseX128;
  constexpr int VST = kXVPF + 1;
  u32x4 (&pf)[4] = xp.pf;
  u32x2 (&vf)[VST][2] = xp.vf;
  auto vread = [&](auto pc, auto hc) {
    constexpr int pp = decltype(pc)::value, h = decltype(hc)::value;
    vf[pp % VST][h] = ds_read_tr16_b64<16 * kRowStride * h + 32 * (pp % 8)>(vrow);
  };
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(xp.fl), "+v"(xp.e) : "n"(Px::kPro - 2));
  const uint32_t fl = xp.fl;
  if (__ballot(fl != 0u) != 0ull) {
    // some wave moved references: rescale what earlier tiles accumulated for
    // its heads (head block o belongs to wave o / 2)
    u32x4 f0 = ds_read_b128<0>(fac_rd);
    u32x4 f1 = ds_read_b128<16>(fac_rd);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f0), "+v"(f1));
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // MFMA write -> accumulator read distance
    static_for<0, 8>([&](auto oc) {
      constexpr int o = decltype(oc)::value;
      const float fo = __uint_as_float(o < 4 ? f0[o] : f1[o - 4]);
      if (__ballot(((fl >> (8 * (o / 2))) & 0xffu) != 0u && fo != 1.f) != 0ull)
        static_for<0, 8>([&](auto dc) { acc128_scale<32 * o + 4 * decltype(dc)::value>(fo); });
    });
    asm volatile("s_nop 4" ::: "memory");  // accumulators rescaled by VALU, read by the MFMAs below
  }
  SoftT tt;
  Deps dep{c, c};
  constexpr int NG = kSoftGroups128<MASK>;
  static_for<0, 16>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    constexpr int dt = u % 8, o0 = 4 * (u / 8);
    if constexpr (u == 0 || u == 8)
      asm volatile("s_waitcnt lgkmcnt(%6)"
                   : "+v"(vf[u % VST][0]), "+v"(vf[u % VST][1]), "+v"(pf[0]), "+v"(pf[1]), "+v"(pf[2]), "+v"(pf[3])
                   : "n"(Px::wait_at(u)));
    else
      asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(vf[u % VST][0]), "+v"(vf[u % VST][1]) : "n"(Px::wait_at(u)));
    const bf16x8 va =
        __builtin_bit_cast(bf16x8, u32x4{vf[u % VST][0][0], vf[u % VST][0][1], vf[u % VST][1][0], vf[u % VST][1][1]});
    static_for<0, 4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      acc128_mfma<32 * (o0 + i) + 4 * dt>(va, __builtin_bit_cast(bf16x8, pf[i]), dep.d0, dep.d1);
      if constexpr (u + kXVPF < 16 && i < 2) vread(Int<u + kXVPF>{}, Int<i>{});
      // the second pass's P fragment replaces this one after its last reader
      if constexpr (u == 7) pf[i] = ds_read_b128<1024 * (4 + i)>(pbase);
      constexpr int G = soft_group_at<NG>(4 * u + i);
      if constexpr (SOFT && G >= 0) dep = soft128_group<G, MASK>(s, tt, ss, c, inv_c, cnt, g, pbw, facw, flagw);
    });
    __builtin_amdgcn_sched_barrier(0);
  });
}

// The 128-head kernel is persistent: workgroup b of G owns one unit (token,
// head group of 128) of every run of G, unit r G + slot_r(b) in run r. Unit v
// is token T - 1 - v / head_groups, head group v % head_groups. Workgroups are
// dispatched to the kNumXcd XCDs in turn, so workgroup b = x + kNumXcd c runs
// on XCD x; when G is a multiple of kNumXcd, the slots of run r that XCD x
// holds are the consecutive x G / kNumXcd .. + G / kNumXcd - 1 (c, or its
// mirror for odd r), so that its CUs work on neighbouring tokens at once and
// share their sliding-window rows in that XCD's L2. The alternating order
// evens out the drift of the weights within a run. The workgroups of XCD x
// take their K runs starting at run x K / kNumXcd and wrapping around, so
// that the XCDs do not all reach a unit's end (128 KiB of output stores per
// workgroup) at the same time.
struct Sched128 {
  int b, G, K, r0, x, c, per;
  __device__ __forceinline__ int slot(int r) const {
    if (per == 0) return (r & 1) ? G - 1 - b : b;
    return x * per + ((r & 1) ? per - 1 - c : c);
  }
  __device__ __forceinline__ Sched128(int b_, int G_, int units) : b(b_), G(G_) {
    per = (G % kNumXcd == 0) ? G / kNumXcd : 0;
    x = b % kNumXcd;
    c = b / kNumXcd;
    const int full = units / G, rem = units % G;
    K = full + ((rem > 0 && slot(full) < rem) ? 1 : 0);
    r0 = K > 0 ? (per == 0 ? b % K : (x * K / kNumXcd) % K) : 0;
  }
  // the unit taken i-th (i < K)
  __device__ __forceinline__ int unit(int i) const {
    int r = r0 + i;
    r = r >= K ? r - K : r;
    return r * G + slot(r);
  }
};

// The top-k entries of a unit are moved into a list buffer by LDS-DMA (wave w
// moves positions 256 c + 64 w + lane, and later reads them back), then
// compacted in place. Positions past len read entry len - 1 (dropped by
// compact128); trow holds at least one entry.
__device__ __forceinline__ void raw128_dma(uint32_t list_lds, const int32_t* trow, int len, int lane, int w) {
#pragma unroll
  for (int c = 0; c < k128Cap / 256; ++c) {
    const int pos = c * 256 + w * 64 + lane;
    __builtin_amdgcn_global_load_lds(trow + max(min(pos, len - 1), 0),
                                     (LDS_AS void*)(uintptr_t)(list_lds + 4 * (c * 256 + w * 64)), 4, 0, 0);
  }
}
// Compacts the valid entries (position < len, slot < nkv) of a list buffer in
// place, order kept; returns the count. Every read precedes the first barrier
// and every write follows it. The DMA that filled the buffer has completed.
__device__ __forceinline__ int compact128(uint32_t list_lds, int len, uint32_t nkv, uint32_t wcnt_lds, int lane, int w) {
  constexpr int NC = k128Cap / 256;
  int raw[NC];
  uint64_t bal[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int pos = c * 256 + w * 64 + lane;
    // (asm: the entries came by DMA, waited for by the caller)
    asm volatile("ds_read_b32 %0, %1" : "=v"(raw[c]) : "v"(list_lds + 4 * pos));
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    asm volatile("" : "+v"(raw[c]));
    const int pos = c * 256 + w * 64 + lane;
    bal[c] = __ballot(pos < len && (uint32_t)raw[c] < nkv);
  }
  if (lane == 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) *(LDS_AS int32_t*)(uintptr_t)(wcnt_lds + 4 * (c * 4 + w)) = __popcll(bal[c]);
  }
  lds_barrier();
  int base = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = __builtin_amdgcn_readfirstlane(*(LDS_AS const int32_t*)(uintptr_t)(wcnt_lds + 4 * (c * 4 + i)));
      off += (i < w) ? ci : 0;
      tot += ci;
    }
    if ((bal[c] >> lane) & 1ull) *(LDS_AS int32_t*)(uintptr_t)(list_lds + 4 * (base + off + lane_rank(bal[c]))) = raw[c];
    base += tot;
  }
  lds_barrier();
  return __builtin_amdgcn_readfirstlane(base);
}

// The output rows of head block O (heads 16 O + li) from the accumulators:
// tuple acc(O, dt) holds, in lane (li, g), d = 128 w + 16 dt + 4 g .. + 4. Two
// tuples (dt, dt + 1) are scaled and rounded, then the odd 16-lane rows of the
// first are exchanged with the even rows of the second, after which lane
// (li, g) holds eight consecutive d, 16 (dt + (g & 1)) + 8 (g >> 1) .. + 8, of
// one of them: one 16 B store, 64 contiguous bytes per head and tuple pair.
template <int O>
__device__ __forceinline__ void store128_block(uint16_t* orow, bool ok, float fo, int g) {
  f32x4 a[8];  // all eight tuples first: the reads are ordered asm, the arithmetic then overlaps
  static_for<0, 8>([&](auto dc) { a[decltype(dc)::value] = acc128_read<32 * O + 4 * decltype(dc)::value>(); });
  static_for<0, 4>([&](auto pc) {
    constexpr int dt = 2 * decltype(pc)::value;
    const f32x4 x = a[dt] * fo;
    const f32x4 y = a[dt + 1] * fo;
    const auto s0 = __builtin_amdgcn_permlane16_swap(bf16pair(x[0], x[1]), bf16pair(y[0], y[1]), false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(bf16pair(x[2], x[3]), bf16pair(y[2], y[3]), false, false);
    const u32x4 v = u32x4{s0[0], s1[0], s0[1], s1[1]};
    if (ok) *(u32x4*)(orow + 16 * (dt + (g & 1)) + 8 * (g >> 1)) = v;
  });
}

template <bool NEG>
__device__ __forceinline__ void smla_fwd128_body(const Params& p) {
  __shared__ __attribute__((aligned(16))) Smem128 sm;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int li = lane & 15;
  const int nwg = gridDim.x, b = blockIdx.x;
  const int units = p.T * p.head_groups;

  // exchange addresses (tile parity par: + par * the buffer size): P of head
  // block o at pbuf + 1024 o + 16 lane; the factor of head 16 o + li at
  // fac + 4 (8 li + o); wave w's flag at byte flag + w
  const uint32_t pb0 = lds_addr(sm.pbuf[0]) + 16 * lane;
  const uint32_t fac0 = lds_addr(sm.fac[0]) + 32 * li;
  const uint32_t flag0 = lds_addr(sm.flag[0]);
  constexpr uint32_t kPbPar = sizeof(sm.pbuf[0]), kFacPar = sizeof(sm.fac[0]), kFlagPar = sizeof(sm.flag[0]);
  const uint32_t pb_own = pb0 + 2048 * w;  // head blocks 2w, 2w + 1
  const uint32_t fac_own = fac0 + 8 * w;   // entries 8 li + 2w, + 1
  const uint32_t flag_own = flag0 + w;
  const uint32_t wcnt = lds_addr(sm.wcnt);

  // logits c * S with c > 0: a negative scale is carried by q (negation is exact)
  const float c = NEG ? -p.scale_log2 : p.scale_log2;
  const float inv_c = 1.f / c;
  const int len = p.topk_n;  // <= k128Cap: one segment per unit
  auto trow_of = [&](int t) {  // any valid address when there are no entries
    return len > 0 ? p.topk + (size_t)t * len : (const int32_t*)(const void*)p.q;
  };
  auto token_of = [&](int v) { return p.T - 1 - v / p.head_groups; };
  auto hbase_of = [&](int v) { return (v % p.head_groups) * 128; };
  const uint16_t* kvp = p.kv;

  // first unit: its entries, q, the next unit's entries; compaction waits for
  // the first four loads only (loads land in issue order)
  const Sched128 sched(b, nwg, units);  // K >= 1: the grid is no larger than the units
  int v = sched.unit(0);
  int t = token_of(v), hbase = hbase_of(v);
  raw128_dma(lds_addr(sm.list[0]), trow_of(t), len, lane, w);
  bf16x8 qf[2][16];
  load_q_any(qf[0], p, t, hbase + 32 * w + li, g);
  load_q_any(qf[1], p, t, hbase + 32 * w + 16 + li, g);
  const bool two = sched.K > 1;
  if (two) raw128_dma(lds_addr(sm.list[1]), trow_of(token_of(sched.unit(1))), len, lane, w);
  acc128_claim_and_zero();
  // issued: 4 list loads, 32 q loads (, 4 loads of the next list)
  if (two) asm volatile("s_waitcnt vmcnt(36)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  int n = compact128(lds_addr(sm.list[0]), len, p.nkv, wcnt, lane, w);
#pragma unroll
  for (int i = 0; i < k128Ahead; ++i)
    gather128(sm.list[0], i, n, i < (n + kBK - 1) / kBK, sm.tile(i), kvp, lane, w).all(lane);

  Soft128 ss;
  for (int r = 0;; ++r) {
    // unit v (token t, heads hbase ..): list r & 1 compacted (n entries), its
    // tiles 0..2 and q issued
    const int32_t* lst = sm.list[r & 1];
    const int nt = (n + kBK - 1) / kBK;
    const bool more = r + 1 < sched.K;
    const int vn = more ? sched.unit(r + 1) : 0;
    const int tn = more ? token_of(vn) : 0, hbn = more ? hbase_of(vn) : 0;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      ss.l_part[hb] = 0.f;
      ss.nmu[hb] = 0.f;
      ss.thr[hb] = -INFINITY;
    }
    // the sinks of this lane's two heads, loaded here so that the boundary
    // does not wait for them behind the next q
    float sk[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int head = hbase + 32 * w + 16 * hb + li;
      sk[hb] = (p.sink != nullptr && head < p.H) ? p.sink[head] : -INFINITY;
    }
    wait_vmcnt_le(0);  // q and tiles 0..2 (and the previous unit's stores)
    asm volatile("" : "+v"(sk[0]), "+v"(sk[1]));
    lds_barrier();
    if constexpr (NEG) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int k = 0; k < 16; ++k)
          qf[hb][k] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf[hb][k]) ^ 0x80008000u);
    }
    f32x4 s[2][2];
    XPre xp;
    // phase X of tile j: accumulates P.V(j); SOFT: with the softmax of tile
    // j + 1 between its MFMAs (MASK: tile j + 1 is the partial last one)
    auto phase_x = [&](int j, auto soft, auto mask) {
      const uint32_t par = j & 1, nxt = par ^ 1;
      const uint32_t vrow = v_frag_addr(sm.tile(j % k128Ring), g, li) + 256 * w;
      const uint32_t pbase = pb0 + kPbPar * par, fac_rd = fac0 + kFacPar * par;
      const uint32_t pbw = pb_own + kPbPar * nxt, facw = fac_own + kFacPar * nxt, flagw = flag_own + kFlagPar * nxt;
      phase_x128<decltype(soft)::value, decltype(mask)::value>(xp, vrow, pbase, fac_rd, s, ss, c, inv_c,
                                                              decltype(mask)::value ? tile_rows(j + 1, n) : kBK, g,
                                                              pbw, facw, flagw);
    };
    // the first reads of phase X(j): tile j, P(j), the flags of tile j, and
    // the list entry of the gather of tile j + 3
    auto prefetch_x = [&](int j) {
      const uint32_t par = j & 1;
      x_prefetch(xp, lst, j + k128Ahead, lane, w, flag0 + kFlagPar * par, pb0 + kPbPar * par,
                 v_frag_addr(sm.tile(j % k128Ring), g, li) + 256 * w);
    };
    if (nt > 0) {
      const NoGather none;
      // S(0), its softmax (P(0) in parity 0), S(1)
      phase_y128(k_frag_addr(sm.tile(0), g, li), qf, s, none, lane);
      if (nt > 1) {
        soft128_plain<false>(s, ss, c, inv_c, kBK, g, pb_own, fac_own, flag_own);
        phase_y128(k_frag_addr(sm.tile(1), g, li), qf, s, none, lane);
      } else {
        soft128_plain<true>(s, ss, c, inv_c, tile_rows(0, n), g, pb_own, fac_own, flag_own);
      }
      lds_barrier();  // P(0) visible
      prefetch_x(0);
      // Iteration j: phase X(j) with the softmax of tile j+1 (full) between
      // its MFMAs; one barrier (P(j+1) and tile j+2 visible, tile j-1 free);
      // phase Y computes S(j+2) and gathers tile j+3 into tile j-1's slot, and
      // issues the first reads of phase X(j+1) behind its last MFMA.
      for (int j = 0; j + 2 < nt; ++j) {
        phase_x(j, std::true_type{}, std::false_type{});
        const uint32_t e = xp.e;  // list entry of tile j + 3 (completed in phase X)
        wait_vmcnt_le(0);         // tile j + 2 landed (issued in phase Y of iteration j - 1)
        lds_barrier();
        const Gather128 ga = gather128_make(e, j + k128Ahead, n, j + k128Ahead < nt,
                                            sm.tile((j + k128Ahead) % k128Ring), kvp, lane, w);
        phase_y128(k_frag_addr(sm.tile((j + 2) % k128Ring), g, li), qf, s, ga, lane, [&]() { prefetch_x(j + 1); });
      }
    }
    // every S of this unit is done: q of the next unit (this unit's again for
    // the last, unused) lands under the last two phases X and the boundary
    load_q_any(qf[0], p, more ? tn : t, (more ? hbn : hbase) + 32 * w + li, g);
    load_q_any(qf[1], p, more ? tn : t, (more ? hbn : hbase) + 32 * w + 16 + li, g);
    if (nt > 1) {  // X(nt - 2) with the softmax of the last tile; nothing more to wait for
      phase_x(nt - 2, std::true_type{}, std::true_type{});
      lds_barrier();
      prefetch_x(nt - 1);
    }
    if (nt > 0) {
      phase_x(nt - 1, std::false_type{}, std::false_type{});
      lds_barrier();
    }

    // ---- unit boundary: lse and output scales of this unit; the next unit's
    // list compacted and its first tiles issued; this unit's rows stored ----
    {
      const int hs = hbase + 32 * w + li;
      float oscale[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int head = hs + 16 * hb;
        const bool has_sink = !(sk[hb] == -INFINITY);
        const HeadEnd he = head_end(ss.l_part[hb], ss.m_ref(hb), sk[hb], has_sink, sk[hb] * kLog2e);
        if (g == 0 && head < p.H) p.lse[(size_t)t * p.H + head] = he.lse;
        oscale[hb] = he.oscale * p.out_scale;  // 1, or an fp8 pool's dequant scale
      }
      const uint32_t osc_own = lds_addr(sm.osc) + 32 * li + 8 * w;
      if (g == 0) {
        *(LDS_AS float*)(uintptr_t)(osc_own) = oscale[0];
        *(LDS_AS float*)(uintptr_t)(osc_own + 4) = oscale[1];
      }
    }
    // output scales visible after the first barrier of the compaction
    const int nn = more ? compact128(lds_addr(sm.list[(r + 1) & 1]), len, p.nkv, wcnt, lane, w) : 0;
    if (!more) lds_barrier();
    u32x4 f0 = ds_read_b128<0>(lds_addr(sm.osc) + 32 * li);
    u32x4 f1 = ds_read_b128<16>(lds_addr(sm.osc) + 32 * li);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f0), "+v"(f1));
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // MFMA write -> accumulator read distance
    {
      uint16_t* orow = p.out + ((size_t)t * p.H + hbase + li) * kD + 128 * w;
      static_for<0, 8>([&](auto oc) {
        constexpr int o = decltype(oc)::value;
        const float fo = __uint_as_float(o < 4 ? f0[o] : f1[o - 4]);
        store128_block<o>(orow + (size_t)16 * o * kD, hbase + 16 * o + li < p.H, fo, g);
      });
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < k128Ahead; ++i)
        gather128(sm.list[(r + 1) & 1], i, nn, i < (nn + kBK - 1) / kBK, sm.tile(i), kvp, lane, w).all(lane);
      if (r + 2 < sched.K)  // into this unit's list buffer, read no more
        raw128_dma(lds_addr(sm.list[r & 1]), trow_of(token_of(sched.unit(r + 2))), len, lane, w);
    }
    acc128_claim_and_zero();
    if (!more) break;
    v = vn;
    t = tn;
    hbase = hbn;
    n = nn;
  }
}

// NEG: the scale is negative (carried by q, negated at load)
template <bool NEG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void smla_fwd128_kernel(const Params p) {
  smla_fwd128_body<NEG>(p);
}

// ---------------------------------------------------------------------------
// H <= 16, bf16 pool: 16-row tiles, one wave of 16 heads per workgroup. A
// 32-row ring of two tiles takes 74 KiB, so only two one-wave workgroups fit
// a CU and two of its four SIMDs hold a wave; with 16-row tiles the ring of
// NBUF tiles and a list of CAP entries take 38 KiB (NBUF 2, CAP 1024: four
// per CU, one wave per SIMD) or 19 KiB (NBUF 1, CAP 640: eight per CU, two
// waves per SIMD). S^T is one 16-row half of the 32-row form; P.V uses the
// 16x16x16 MFMA, whose A operand is one transposing read and whose B operand
// is the four P values the S^T accumulator layout leaves in each lane.

template <int NBUF, int CAP, bool FP8 = false>
struct Smem16 {
  static constexpr int kTileBytes = FP8 ? kBK16 * kD : kBK16 * kRowStride;
  static constexpr int kRing = NBUF * kTileBytes;
  static constexpr int kStage = 16 * kRowStride;
  static constexpr int kAreaBytes = kRing > kStage ? kRing : kStage;
  uint8_t area[kAreaBytes];
  int32_t list[CAP];
  __device__ __forceinline__ uint32_t tile(int b) { return lds_addr(area + b * kTileBytes); }
  __device__ __forceinline__ uint32_t stage() { return lds_addr(area); }
};

// S^T = K Q^T for a 16-row tile: s holds S^T[slot 4g + i][head li]. Four
// independent MFMA chains (k mod 4), summed at the end.
template <int KPF>
__device__ __forceinline__ void tile_s16(uint32_t krow, const bf16x8 (&qf)[16], f32x4& s) {
  constexpr int KST = KPF + 1;
  f32x4 sp[4];
  u32x4 kf[KST];
  auto kread = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    kf[k % KST] = ds_read_b128<64 * k>(krow);
  };
  static_for<0, KPF>([&](auto kc) { kread(kc); });
  static_for<0, 16>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k + KPF < 16) kread(Int<k + KPF>{});
    constexpr int younger = 15 - k < KPF ? 15 - k : KPF;
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(kf[k % KST]) : "n"(younger));
    if constexpr (k < 4) mfma_s_first(sp[k & 3], kf[k % KST], __builtin_bit_cast(u32x4, qf[k]));
    else mfma_s(sp[k & 3], kf[k % KST], __builtin_bit_cast(u32x4, qf[k]));
    __builtin_amdgcn_sched_barrier(0);
  });
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // MFMA write -> VALU read distance
  asm volatile("" : "+v"(sp[0]), "+v"(sp[1]), "+v"(sp[2]), "+v"(sp[3]));
  s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
}

// Online softmax of a 16-row tile (as tile_softmax, four slots per lane).
__device__ __forceinline__ void tile_softmax16(const f32x4& s, int cnt, float scale_log2, int g, float& m_ref,
                                               float& l_part, f32x4 (&acc)[32], bf16x4& pk) {
  float x[4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float xv = 4 * g + i < cnt ? s[i] * scale_log2 : -INFINITY;
    x[i] = xv;
    mx = __builtin_fmaxf(mx, xv);
  }
  mx = row4_max(mx);
  if (__ballot(mx > m_ref + kLazyTau) != 0ull) {
    const float m_new = __builtin_fmaxf(m_ref, mx);
    if (__ballot(m_ref != -INFINITY) != 0ull) {
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_part *= alpha;
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
  for (int i = 0; i < 4; ++i) {
    const float pv = __builtin_amdgcn_exp2f(x[i] - mu);
    ls += pv;
    pk[i] = (__bf16)pv;
  }
  l_part += ls;
}

// ---- 16-row tiles of an fp8 pool ----
// Tile layout, slab-major: block k (512 bytes) holds d = 32k .. 32k+31 of the 16
// rows as two 16-byte chunks per row, chunk j of row r at 16 (r + 16 j). One
// LDS-DMA instruction fills blocks 2m and 2m+1 (lane L: row L % 16, chunk
// (L / 16) % 2 of block 2m + L / 32, written at byte 16 L), so a tile takes 8
// instructions; rows past the tile's count come from a zero row.
struct TileIssue8r16 {
  const uint8_t* src;  // this lane's bytes of its row in blocks 0 and 1
  uint32_t dst0;
  bool act;
  __device__ __forceinline__ void init(const int32_t* list, int i, int n, bool act_, uint32_t buf, const uint8_t* kv,
                                       int lane, int w) {
    (void)w;
    act = act_;
    dst0 = buf;
    const int cnt = act ? min(kBK16, n - i * kBK16) : 0;
    const int row = lane & 15;
    const bool valid = act && row < cnt;
    uint32_t e = 0;
    if (valid) asm volatile("ds_read_b32 %0, %1" : "=v"(e) : "v"(lds_addr(list + i * kBK16 + row)));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(e));
    const uint8_t* base = valid ? uniform_ptr(kv) + ((uint64_t)e << 9) : uniform_ptr(kZeroRow8);
    src = base + 32 * (lane >> 5) + 16 * ((lane >> 4) & 1);
  }
  __device__ __forceinline__ void all(int lane) const {
    (void)lane;
    if (!act) return;
    static_for<0, 8>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      __builtin_amdgcn_global_load_lds(src + 64 * m, (LDS_AS void*)(uintptr_t)(dst0 + 1024 * m), 16, 0, 0);
    });
  }
};

// S^T = K Q^T for a 16-row fp8 tile: the K fragment of k-step k (lane: row li,
// d = 32k + 8g .. +8) is 8 bytes at kaddr + 512 k, kaddr = tile + 16 (li + 16 (g / 2))
// + 8 (g % 2), converted to bf16 before the MFMA. Four chains (k mod 4).
template <int KPF>
__device__ __forceinline__ void tile_s8r16(uint32_t kaddr, const bf16x8 (&qf)[16], f32x4& s) {
  constexpr int KST = KPF + 1;
  f32x4 sp[4];
  u32x2 kf[KST];
  auto kread = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    kf[k % KST] = ds_read_b64<512 * k>(kaddr);
  };
  // k-step k's fragment is converted during step k - 1, so that the asm
  // conversions (VALU) sit several instructions before their MFMA reader;
  // only the last step's reader needs explicit wait states.
  static_for<0, KPF>([&](auto kc) { kread(kc); });
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(kf[0]) : "n"(KPF - 1));
  u32x4 acur = fp8x8_to_bf16(kf[0]);
  asm volatile("" : "+v"(acur));  // converted above step 0's reads and conversion
  static_for<0, 16>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k + KPF < 16) kread(Int<k + KPF>{});
    u32x4 anext;
    if constexpr (k + 1 < 16) {
      constexpr int younger = 14 - k < KPF - 1 ? 14 - k : KPF - 1;  // reads issued after step k+1's
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(kf[(k + 1) % KST]) : "n"(younger));
      anext = fp8x8_to_bf16(kf[(k + 1) % KST]);
      asm volatile("" : "+v"(anext));  // the conversion stays above this step's MFMA
    } else {
      valu_to_mfma(acur);  // no conversion between the last one and its reader
    }
    if constexpr (k < 4) mfma_s_first(sp[k & 3], acur, __builtin_bit_cast(u32x4, qf[k]));
    else mfma_s(sp[k & 3], acur, __builtin_bit_cast(u32x4, qf[k]));
    if constexpr (k + 1 < 16) acur = anext;
    __builtin_amdgcn_sched_barrier(0);
  });
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // MFMA write -> VALU read distance
  asm volatile("" : "+v"(sp[0]), "+v"(sp[1]), "+v"(sp[2]), "+v"(sp[3]));
  s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
}

// V^T fragment base of a 16-row fp8 tile for the 16x16x16 MFMA: lane
// (g, li) must end up with V[4g .. 4g+3][16 dt + li]. In the transposing 8-bit
// read, lane li of a 16-lane group receives byte li % 8 of the fetches of
// lanes 2m + li / 8 (m = 0..7); lane 2m + h therefore fetches row 4g + (m % 4)
// at columns 8h .. 8h+7 of the d-tile, and the low four bytes received are
// slots 4g .. 4g+3 (the high four repeat them and are not used).
__device__ __forceinline__ uint32_t v8r16_frag_addr(uint32_t tile, int g, int li) {
  const int m = li >> 1;
  return opaque(tile + 16 * (4 * g + (m & 3)) + 8 * (li & 1));
}

// O^T += V^T P^T for a 16-row fp8 tile: d-tile dt is one transposing read at
// vaddr + 512 (dt / 2) + 256 (dt % 2), four codes converted to bf16.
__device__ __forceinline__ void tile_pv8r16(uint32_t vaddr, const bf16x4& pk, f32x4 (&acc)[32]) {
  asm volatile("s_nop 4" ::: "memory");  // P written by VALU, read by MFMA below
  constexpr int VPF = 6;
  constexpr int VST = VPF + 1;
  const u32x2 pb = __builtin_bit_cast(u32x2, pk);
  u32x2 vf[VST];
  auto vread = [&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    vf[dt % VST] = ds_read_tr8_b64<512 * (dt / 2) + 256 * (dt % 2)>(vaddr);
  };
  // d-tile dt's fragment is converted during d-tile dt - 1 (see tile_s8r16)
  static_for<0, VPF>([&](auto dc) { vread(dc); });
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(vf[0]) : "n"(VPF - 1));
  u32x2 acur = u32x2{fp8x2_to_bf16<false>(vf[0][0]), fp8x2_to_bf16<true>(vf[0][0])};
  asm volatile("" : "+v"(acur));
  static_for<0, 32>([&](auto dc) {
    constexpr int dt = decltype(dc)::value;
    if constexpr (dt + VPF < 32) vread(Int<dt + VPF>{});
    u32x2 anext;
    if constexpr (dt + 1 < 32) {
      constexpr int younger = 30 - dt < VPF - 1 ? 30 - dt : VPF - 1;  // reads issued after d-tile dt+1's
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(vf[(dt + 1) % VST]) : "n"(younger));
      anext = u32x2{fp8x2_to_bf16<false>(vf[(dt + 1) % VST][0]), fp8x2_to_bf16<true>(vf[(dt + 1) % VST][0])};
      asm volatile("" : "+v"(anext));  // the conversion stays above this d-tile's MFMA
    } else {
      asm volatile("s_nop 3" : "+v"(acur));  // no conversion between the last one and its reader
    }
    mfma16_acc(acc[dt], acur, pb);
    if constexpr (dt + 1 < 32) acur = anext;
    __builtin_amdgcn_sched_barrier(0);
  });
}

// One workgroup (one wave) per token. Tile j+NBUF-1 is gathered at the top of
// iteration j (its ring slot was last read in iteration j-1, whose reads have
// completed), then the wave waits for tile j and computes it.
template <int NBUF, int CAP, bool FP8, bool I64 = false>
__device__ __forceinline__ void smla_fwd16_body(const Params& p) {
  static_assert(NBUF == 1 || NBUF == 2, "ring of one or two 16-row tiles");
  static_assert(!(I64 && FP8), "int64 rows are read directly by the bf16 kernel only");
  static_assert(FP8 || NBUF == 1, "a bf16 pool runs one tile at a time (the next tile's list entries are read ahead)");
  constexpr int AHEAD = NBUF - 1;
  using SM = Smem16<NBUF, CAP, FP8>;
  __shared__ __attribute__((aligned(16))) SM sm;

  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;
  const int t = p.T - 1 - xcd_remap(blockIdx.x, gridDim.x);  // latest (heaviest) tokens first
  const int head = li;

  f32x4 acc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_part = 0.f;
  bf16x8 qf[16];
  load_q(qf, p, t, head, g);
  bf16x4 pk;

  using Idx = typename std::conditional<I64, int64_t, int32_t>::type;
  const Idx* trow;
  if constexpr (I64) trow = p.topk64 + (size_t)t * p.topk_n;
  else trow = p.topk + (size_t)t * p.topk_n;
  using Issue = typename std::conditional<FP8, TileIssue8r16, TileIssue<1, kBK16>>::type;
  using Elem = typename std::conditional<FP8, uint8_t, uint16_t>::type;
  const Elem* kvp = (const Elem*)p.kv;
  constexpr int kDma = FP8 ? 8 : kBK16;  // LDS-DMA instructions per tile
  for (int seg0 = 0; seg0 < p.topk_n; seg0 += CAP) {
    const int n = compact_segment<1, SM, CAP>(trow + seg0, min(CAP, p.topk_n - seg0), p.nkv, sm, lane, 0);
    const int ntiles = (n + kBK16 - 1) / kBK16;
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
      Issue is;
      is.init(sm.list, i, n, i < ntiles, sm.tile(i), kvp, lane, 0);
      is.all(lane);
    }
    // bf16 (one tile in flight): the list entries and row addresses of tile
    // j + 1 are formed during tile j, so that its gather issues at once
    typename TileIssue<1, kBK16>::Rows rw{};
    TileIssue<1, kBK16> nx{};
    if constexpr (!FP8) {
      nx.init(sm.list, 0, n, true, sm.tile(0), p.kv, lane, 0);
      nx.rows(rw);
    }
    for (int j = 0; j < ntiles; ++j) {
      const bool ahead = j + AHEAD < ntiles;
      if constexpr (FP8) {
        Issue is;
        is.init(sm.list, j + AHEAD, n, ahead, sm.tile((j + AHEAD) % NBUF), kvp, lane, 0);
        is.all(lane);
      } else {
        nx.issue(rw, lane);
      }
      int e_next = 0;
      if constexpr (!FP8) e_next = sm.list[min((j + 1) * kBK16 + li, CAP - 1)];
      wait_vmcnt_le(AHEAD > 0 && ahead ? kDma : 0);  // tile j landed (tile j + AHEAD may be in flight)
      const uint32_t tb = sm.tile(j % NBUF);
      f32x4 sv;
      if constexpr (FP8) tile_s8r16<3>(opaque(tb + 16 * (li + 16 * (g >> 1)) + 8 * (g & 1)), qf, sv);
      else tile_s16<3>(k_frag_addr(tb, g, li), qf, sv);
      tile_softmax16(sv, min(kBK16, n - j * kBK16), p.scale_log2, g, m_ref, l_part, acc, pk);
      if constexpr (!FP8) {
        nx.init_with(e_next, j + 1, n, j + 1 < ntiles, sm.tile(0), p.kv, lane, 0);
        nx.rows(rw);
      }
      if constexpr (FP8) tile_pv8r16(v8r16_frag_addr(tb, g, li), pk, acc);
      else tile_pv16(v_frag_addr(tb, g, li), pk, acc);
    }
  }

  // finalise: fold the sink, normalise, stage 16 rows, store whole rows
  const float sk = (p.sink != nullptr && head < p.H) ? p.sink[head] : -INFINITY;
  const bool has_sink = !(sk == -INFINITY);
  const float sink_l2 = sk * kLog2e;
  HeadEnd he = head_end(l_part, m_ref, sk, has_sink, sink_l2);
  he.oscale *= p.out_scale;  // 1, or the dequant scale of an fp8 pool (V == code * scale)
  if (g == 0 && head < p.H) p.lse[(size_t)t * p.H + head] = he.lse;
  const uint32_t ob = sm.stage();
  mfma_agpr_drain(acc);
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) {
    const f32x4 o = acc[dt] * he.oscale;
    const bf16x4 ob4 = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
    *(LDS_AS bf16x4*)(uintptr_t)(ob + li * kRowStride + 32 * dt + 8 * g) = ob4;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const u32x4 val = *(LDS_AS const u32x4*)(uintptr_t)(ob + r * kRowStride + 16 * lane);
    if (r < p.H) __builtin_nontemporal_store(val, (u32x4*)(p.out + ((size_t)t * p.H + r) * kD + 8 * lane));
  }
}

template <int NBUF, int CAP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NBUF == 1 ? 2 : 1))) void smla_fwd16_kernel(
    const Params p) {
  smla_fwd16_body<NBUF, CAP, false>(p);
}

// The same for a pool of OCP FP8 E4M3 codes: 8 KiB tiles, so a ring of two
// still fits the 16.5 KiB output staging area (19 KiB of LDS, eight per CU).
template <int NBUF, int CAP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void smla_fwd16_fp8_kernel(const Params p) {
  smla_fwd16_body<NBUF, CAP, true>(p);
}

// The bf16 16-row kernel on int64 top-k rows: the compaction tests each entry
// in 64 bits and narrows the valid ones, so no conversion pass precedes it.
template <int CAP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void smla_fwd16_i64_kernel(const Params p) {
  smla_fwd16_body<1, CAP, false, true>(p);
}

// Merge of the splits of one (token, head), one wave each: lane s < nsplit
// reads split s's reference max m_s and sum l_s; with Mv the largest m_s, the
// splits are weighted by c_s = 2^(m_s - Mv) (0 for a split that saw no valid
// slot), and lane L accumulates o[t, h, 8L .. 8L+8). The sink is then folded in
// exactly as in the single-pass finalisation.
__global__ __launch_bounds__(256) void smla_merge_kernel(const Params p, const SplitArgs sa, int heads_per_group) {
  const int lane = threadIdx.x & 63;
  const int th = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (th >= p.T * p.H) return;
  const int t = th / p.H;
  const int h = th - t * p.H;
  const int hg = h / heads_per_group;
  const int hi = h - hg * heads_per_group;
  const size_t base = ((size_t)(p.T - 1 - t) * p.head_groups + hg) * sa.nsplit * heads_per_group + hi;
  float ms = -INFINITY, ls = 0.f;
  if (lane < sa.nsplit) {
    const size_t pi = base + (size_t)lane * heads_per_group;
    ms = sa.part_ml[2 * pi];
    ls = sa.part_ml[2 * pi + 1];
  }
  const float mv = wave_max(ms);
  const float c = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - mv);
  const float lsum = wave_sum(ls * c);
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int sp = 0; sp < sa.nsplit; ++sp) {
    const float cs = __shfl(c, sp, 64);
    const f32x4* src = (const f32x4*)(sa.part_o + (base + (size_t)sp * heads_per_group) * kD + 8 * lane);
    o0 += src[0] * cs;
    o1 += src[1] * cs;
  }
  const float sk = p.sink != nullptr ? p.sink[h] : -INFINITY;
  const bool has_sink = !(sk == -INFINITY);
  const float sink_l2 = sk * kLog2e;
  uint16_t* dst = p.out + ((size_t)t * p.H + h) * kD + 8 * lane;
  if (lsum == 0.f) {  // no valid slot carried any mass
    *(u32x4*)dst = u32x4{0u, 0u, 0u, 0u};
    if (lane == 0) p.lse[(size_t)t * p.H + h] = has_sink ? sk : -INFINITY;
    return;
  }
  const float mf = has_sink ? __builtin_fmaxf(mv, sink_l2) : mv;
  const float a = __builtin_amdgcn_exp2f(mv - mf);
  const float lf = lsum * a + (has_sink ? __builtin_amdgcn_exp2f(sink_l2 - mf) : 0.f);
  const float oscale = a / lf * p.out_scale;
  o0 *= oscale;
  o1 *= oscale;
  *(bf16x8*)dst = bf16x8{(__bf16)o0[0], (__bf16)o0[1], (__bf16)o0[2], (__bf16)o0[3],
                         (__bf16)o1[0], (__bf16)o1[1], (__bf16)o1[2], (__bf16)o1[3]};
  if (lane == 0) p.lse[(size_t)t * p.H + h] = (mf + __builtin_amdgcn_logf(lf)) * kLn2;
}

struct Variant {
  int nw;
  const char* name;
};

// One wave per 16 heads. Up to 16 heads the single pass runs the 16-row
// kernels (one wave, 19 KiB of LDS, eight workgroups per CU); the 32-row
// one-wave form serves only the few-token split path. A 32-row bf16 tile takes
// 33 KiB: workgroups of 2 or 4 waves with 2 tiles, two per CU; wider heads are
// cut into groups of 64, so that two 4-wave D-split workgroups share a CU and
// one hides the other's gather waits, softmax, barriers and finalisation (each
// row is then gathered once per group; the second gather mostly hits L2). A
// 32-row fp8 tile takes 16 KiB: 2 at two waves, 4 at four waves (in the output
// staging area's room); above 64 heads one 8-wave workgroup of 128 heads with
// 4 tiles, dequantised once into two shared bf16 tiles, so that the conversion
// is not repeated per head group.
// 16-row variant for H <= 16 and a bf16 pool (single pass): one tile and a
// 640-entry list, eight workgroups per CU (a ring of two tiles with a
// 1024-entry list fits four per CU and measured 1.3x slower). 640 entries
// take a 640-slot row in one segment (the second segment's index loads
// stalled the wave: 512 entries were 0.8% slower there).
constexpr int kR16Nbuf = 1;
constexpr int kR16Cap = 640;
// More than 64 heads over a bf16 pool run on the persistent 128-head kernel
// (smla_fwd128_kernel) whenever the top-k row fits its 1024-entry list; longer
// rows take two 64-head workgroups per token of the D-split kernel.
constexpr bool kFwd128 = true;

Variant pick_variant(int64_t H, int64_t topk, bool fp8) {
  if (H <= 16 && !fp8) return {1, "smla_fwd16_kernel<1, 640>"};
  if (H <= 16) return {1, "smla_fwd16_fp8_kernel<2, 512>"};
  if (H <= 32) return {2, fp8 ? "smla_fwd_fp8_kernel<2, 2>" : "smla_fwd_kernel<2, 2>"};
  if (!fp8) return {4, (H > 64 && kFwd128 && topk <= k128Cap) ? "smla_fwd128_kernel" : "smla_fwd_kernel<4, 2>"};
  if (H <= 64) return {4, "smla_fwd_fp8_kernel<4, 4>"};
  return {8, "smla_fwd_fp8_kernel<8, 4>"};
}

template <int NW, int NBUF, bool SPLIT, bool FP8>
hipError_t launch(const Params& p, const SplitArgs& sa, int blocks, hipStream_t stream) {
  if constexpr (SPLIT && FP8) {
    hipLaunchKernelGGL((smla_fwd_fp8_split_kernel<NW, NBUF>), dim3(blocks), dim3(NW * 64), 0, stream, p, sa);
  } else if constexpr (SPLIT) {
    hipLaunchKernelGGL((smla_fwd_split_kernel<NW, NBUF>), dim3(blocks), dim3(NW * 64), 0, stream, p, sa);
  } else if constexpr (FP8) {
    (void)sa;
    hipLaunchKernelGGL((smla_fwd_fp8_kernel<NW, NBUF>), dim3(blocks), dim3(NW * 64), 0, stream, p);
  } else {
    (void)sa;
    hipLaunchKernelGGL((smla_fwd_kernel<NW, NBUF>), dim3(blocks), dim3(NW * 64), 0, stream, p);
  }
  return hipGetLastError();
}

template <bool SPLIT, bool FP8>
hipError_t launch_variant(int nw, const Params& p, const SplitArgs& sa, int blocks, hipStream_t s) {
  if (nw == 1) {
    // the single pass at H <= 16 runs the 16-row kernels (run_prefill)
    if constexpr (SPLIT) return launch<1, 2, SPLIT, FP8>(p, sa, blocks, s);
    return hipErrorInvalidValue;
  }
  if (nw == 2) return launch<2, 2, SPLIT, FP8>(p, sa, blocks, s);
  if (nw == 4) return launch<4, FP8 ? 4 : 2, SPLIT, FP8>(p, sa, blocks, s);
  if constexpr (FP8) return launch<8, 4, SPLIT, FP8>(p, sa, blocks, s);
  return hipErrorInvalidValue;  // bf16 pools use at most 4 waves per workgroup
}

// A split covers at least this many top-k positions (two full tiles); a row
// is split at most kMaxSplit ways (one merge lane per split).
constexpr int kMinSplitLen = 64;
constexpr int kMaxSplit = 64;



// Argument checks shared by the entry points (idx_align: alignment the top-k
// array needs). Everything but the device query.
int check_args(const void* q, const void* kv, const void* topk_indices, size_t idx_align, const float* attn_sink,
               float scale, const void* out, const float* lse, int64_t T, int64_t H, int64_t num_kv, int64_t topk,
               bool fp8) {
  if (T < 0 || H < 1 || num_kv < 0 || topk < 0) return SMLA_ERR_BAD_SIZE;
  if (T > INT32_MAX || H > INT32_MAX || topk > INT32_MAX) return SMLA_ERR_BAD_SIZE;
  if (!isfinite(scale)) return SMLA_ERR_BAD_SCALE;
  if (T == 0) return SMLA_OK;
  const Variant var = pick_variant(H, topk, fp8);
  const int64_t heads_per_wg = (int64_t)16 * var.nw;
  const int64_t head_groups = (H + heads_per_wg - 1) / heads_per_wg;
  if (T * head_groups > INT32_MAX) return SMLA_ERR_BAD_SIZE;
  if (T > INT64_MAX / H / kD || T > INT64_MAX / (topk > 0 ? topk : 1)) return SMLA_ERR_BAD_SIZE;
  if (!q || !out || !lse) return SMLA_ERR_NULL_POINTER;
  if (topk > 0 && !topk_indices) return SMLA_ERR_NULL_POINTER;
  if (topk > 0 && num_kv > 0 && !kv) return SMLA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(out, 16) || (kv && !aligned(kv, 16))) return SMLA_ERR_MISALIGNED;
  if (!aligned(lse, 4) || (topk_indices && !aligned(topk_indices, idx_align)) || (attn_sink && !aligned(attn_sink, 4)))
    return SMLA_ERR_MISALIGNED;
  return SMLA_OK;
}

// Compute units of device dev, looked up once: the grid of a persistent
// kernel (any positive grid is correct; more than one workgroup per CU only
// queues).
int cu_count(int dev) {
  static std::atomic<int> cache[64];
  if (dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Enqueue the forward for int32 top-k rows (arguments already checked, T > 0).
// fixed_ws / fixed_cap: caller-provided scratch for the split path's partials
// (the entry point that allocates nothing); NULL takes them from the pool.
int run_prefill(const void* q, const void* kv, const int32_t* topk_indices, const float* attn_sink, float scale,
                void* out, float* lse, int64_t T, int64_t H, int64_t num_kv, int64_t topk, int dev,
                hipStream_t s, bool fp8 = false, float kv_scale = 1.f, void* fixed_ws = nullptr,
                size_t fixed_cap = 0, const int64_t* topk64 = nullptr) {
  const Variant var = pick_variant(H, topk, fp8);
  const int64_t heads_per_wg = (int64_t)16 * var.nw;
  const int64_t head_groups = (H + heads_per_wg - 1) / heads_per_wg;
  Params p;
  p.q = (const uint16_t*)q;
  p.kv = (const uint16_t*)kv;
  p.topk = topk_indices;
  p.topk64 = topk64;
  p.sink = attn_sink;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.T = (int)T;
  p.H = (int)H;
  p.nkv = (uint32_t)(num_kv < ((int64_t)1 << 31) ? num_kv : ((int64_t)1 << 31));
  if (topk == 0 || !kv) p.nkv = 0;
  // int64 rows are taken only by the single-pass 16-row kernel (the caller checks)
  if (topk64 != nullptr && (H > 16 || fp8)) return SMLA_ERR_BAD_SIZE;
  p.topk_n = (int)topk;
  p.head_groups = (int)head_groups;
  // a pool of fp8 codes (read by the fp8 kernels, or decoded to bf16 code
  // values beforehand) carries its dequant scale here; 1 for a bf16 pool
  p.scale_log2 = scale * kv_scale * kLog2e;
  p.out_scale = kv_scale;
  SplitArgs sa;
  sa.nsplit = 1;
  sa.split_len = (int)topk;
  sa.part_o = nullptr;
  sa.part_ml = nullptr;
  const int64_t units = T * head_groups;

  // Few (token, head group) units leave most CUs idle: split each top-k row
  // over several workgroups, then merge (stream-ordered scratch; if it cannot
  // be had, the single-pass path below still gives the result).
  const int64_t cus = cu_count(dev);
  if (topk64 == nullptr && cus > 0 && units < cus && topk >= 2 * kMinSplitLen) {
    const int64_t slots = (var.nw == 8 ? 1 : 2) * cus;  // resident workgroups
    int64_t ns = (slots + units - 1) / units;
    ns = ns < topk / kMinSplitLen ? ns : topk / kMinSplitLen;
    ns = ns < kMaxSplit ? ns : kMaxSplit;
    if (ns >= 2) {
      const int64_t len = (topk + ns - 1) / ns;
      ns = (topk + len - 1) / len;
      const int64_t parts = units * ns * 16 * var.nw;
      const size_t bytes_o = (size_t)parts * kD * sizeof(float);
      const size_t bytes = bytes_o + (size_t)parts * 2 * sizeof(float);
      void* ws = nullptr;
      const bool pooled = fixed_ws == nullptr;
      if (!pooled) {
        if (bytes > fixed_cap) return SMLA_ERR_SCRATCH_LIMIT;  // nothing enqueued
        ws = fixed_ws;
      } else {
        hipMemPool_t pool = scratch_pool(dev);
        if (pool == nullptr || hipMallocFromPoolAsync(&ws, bytes, pool, s) != hipSuccess) ws = nullptr;
      }
      if (ws != nullptr) {
        sa.nsplit = (int)ns;
        sa.split_len = (int)len;
        sa.part_o = (float*)ws;
        sa.part_ml = (float*)((char*)ws + bytes_o);
        hipError_t err = fp8 ? launch_variant<true, true>(var.nw, p, sa, (int)(units * ns), s)
                             : launch_variant<true, false>(var.nw, p, sa, (int)(units * ns), s);
        if (err == hipSuccess) {
          hipLaunchKernelGGL(smla_merge_kernel, dim3((unsigned)((T * H + 3) / 4)), dim3(256), 0, s, p, sa, 16 * var.nw);
          err = hipGetLastError();
        }
        const hipError_t ferr = pooled ? hipFreeAsync(ws, s) : hipSuccess;
        return (err == hipSuccess && ferr == hipSuccess) ? SMLA_OK : SMLA_ERR_LAUNCH;
      }
      (void)hipGetLastError();
    }
  }
  if (kFwd128 && H > 64 && !fp8 && topk <= k128Cap) {
    p.head_groups = (int)((H + 127) / 128);
    const int64_t units128 = T * p.head_groups;
    const unsigned grid = (unsigned)std::min<int64_t>(units128, cu_count(dev));  // persistent
    if (p.scale_log2 < 0.f)
      hipLaunchKernelGGL(smla_fwd128_kernel<true>, dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(smla_fwd128_kernel<false>, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
  }
  if (H <= 16) {
    if (fp8) hipLaunchKernelGGL((smla_fwd16_fp8_kernel<2, 512>), dim3((unsigned)units), dim3(64), 0, s, p);
    else if (topk64 != nullptr) hipLaunchKernelGGL((smla_fwd16_i64_kernel<kR16Cap>), dim3((unsigned)units), dim3(64), 0, s, p);
    else hipLaunchKernelGGL((smla_fwd16_kernel<kR16Nbuf, kR16Cap>), dim3((unsigned)units), dim3(64), 0, s, p);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
  }
  const hipError_t err = fp8 ? launch_variant<false, true>(var.nw, p, sa, (int)units, s)
                            : launch_variant<false, false>(var.nw, p, sa, (int)units, s);
  return err == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}


// Whether a bf16 call runs the single-pass 16-row kernel: H <= 16 and either
// as many tokens as compute units or rows too short to split (the split
// condition of run_prefill, whose units are the tokens at H <= 16).
bool single_pass16(int64_t T, int64_t H, int64_t topk, int dev) {
  const int64_t cus = cu_count(dev);
  return H <= 16 && !(cus > 0 && T < cus && topk >= 2 * kMinSplitLen);
}


}  // namespace

// ---- scratch of sparse_mla_prefill_noalloc ----
// The split path's partial results for callers that cannot allocate: one
// array per device, held from the library's first use on that device until
// the process ends. Host code never passes `scratch` itself to a kernel (on
// the host the name is only a stand-in for the symbol): it uses the device
// address looked up once per device with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)SPARSE_MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static int noalloc_scratch(int dev, void** ptr) {
  static std::mutex mu;
  static void* addr[64];
  if (dev < 0 || dev >= 64) return SMLA_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return SMLA_ERR_NO_MEMORY;
    }
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return SMLA_OK;
}

extern "C" int sparse_mla_prefill(const void* q, const void* kv, const int32_t* topk_indices, const float* attn_sink,
                                  float scale, void* out, float* lse, int64_t T, int64_t H, int64_t num_kv,
                                  int64_t topk, void* stream) {
  int rc = check_args(q, kv, topk_indices, 4, attn_sink, scale, out, lse, T, H, num_kv, topk, false);
  if (rc != SMLA_OK || T == 0) return rc;
  int dev = -1;
  if ((rc = current_device(&dev)) != SMLA_OK) return rc;
  return run_prefill(q, kv, topk_indices, attn_sink, scale, out, lse, T, H, num_kv, topk, dev, (hipStream_t)stream);
}

extern "C" int sparse_mla_prefill_noalloc(const void* q, const void* kv, const int32_t* topk_indices,
                                          const float* attn_sink, float scale, void* out, float* lse, int64_t T,
                                          int64_t H, int64_t num_kv, int64_t topk, void* stream) {
  int rc = check_args(q, kv, topk_indices, 4, attn_sink, scale, out, lse, T, H, num_kv, topk, false);
  if (rc != SMLA_OK || T == 0) return rc;
  int dev = -1;
  if ((rc = current_device(&dev)) != SMLA_OK) return rc;
  void* ws = nullptr;
  if ((rc = noalloc_scratch(dev, &ws)) != SMLA_OK) return rc;
  return run_prefill(q, kv, topk_indices, attn_sink, scale, out, lse, T, H, num_kv, topk, dev, (hipStream_t)stream,
                     false, 1.f, ws, kNoAllocScratchBytes);
}

// An fp8 call may first decode the whole pool into bf16 scratch and run the
// bf16 kernels on it: a 16-row fp8 tile costs each wave 128 two-code
// conversions per use, more than its halved gather saves, while one decode
// pass moves num_kv * 1.5 KiB. Worth it when the call gathers many times the
// pool's rows (T * topk >= 8 num_kv) and the copy is modest (<= 256 MiB);
// decode-sized calls and very large pools keep the fp8 kernels.
static constexpr int64_t kFp8DecodeMaxRows = ((int64_t)256 << 20) / kRowBytes;
static constexpr int64_t kFp8DecodeMinReuse = 8;
static std::atomic<int> g_fp8_pool_decode{SMLA_FP8_POOL_DECODE_AUTO};

static bool fp8_pool_decoded(int64_t T, int64_t topk, int64_t num_kv) {
  const int mode = g_fp8_pool_decode.load(std::memory_order_relaxed);
  if (mode == SMLA_FP8_POOL_DECODE_NEVER || T <= 0 || topk <= 0 || num_kv <= 0) return false;
  if (mode == SMLA_FP8_POOL_DECODE_ALWAYS) return true;
  return num_kv <= kFp8DecodeMaxRows && kFp8DecodeMinReuse * num_kv <= T * topk;
}

extern "C" int sparse_mla_set_fp8_pool_decode(int mode) {
  if (mode != SMLA_FP8_POOL_DECODE_NEVER && mode != SMLA_FP8_POOL_DECODE_AUTO && mode != SMLA_FP8_POOL_DECODE_ALWAYS)
    return -1;
  return g_fp8_pool_decode.exchange(mode);
}

extern "C" int sparse_mla_fp8_pool_decoded(int64_t T, int64_t topk, int64_t num_kv) {
  return fp8_pool_decoded(T, topk, num_kv) ? 1 : 0;
}

extern "C" int sparse_mla_prefill_fp8(const void* q, const void* kv, float kv_scale, const int32_t* topk_indices,
                                      const float* attn_sink, float scale, void* out, float* lse, int64_t T,
                                      int64_t H, int64_t num_kv, int64_t topk, void* stream) {
  int rc = check_args(q, kv, topk_indices, 4, attn_sink, scale, out, lse, T, H, num_kv, topk, true);
  if (rc != SMLA_OK) return rc;
  if (!isfinite(kv_scale) || !isfinite(scale * kv_scale)) return SMLA_ERR_BAD_SCALE;
  if (T == 0) return SMLA_OK;
  int dev = -1;
  if ((rc = current_device(&dev)) != SMLA_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (fp8_pool_decoded(T, topk, num_kv)) {
    void* ws = nullptr;
    hipMemPool_t pool = scratch_pool(dev);
    if (pool != nullptr && hipMallocFromPoolAsync(&ws, (size_t)num_kv * kRowBytes, pool, s) == hipSuccess &&
        ws != nullptr) {
      const int64_t n16 = num_kv * (kD / 16);
      const int64_t want = (n16 + 255) / 256;
      const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
      hipLaunchKernelGGL(smla_fp8_pool_decode_kernel, dim3(blocks), dim3(256), 0, s, (const uint8_t*)kv,
                         (uint16_t*)ws, n16);
      rc = hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
      if (rc == SMLA_OK)
        rc = run_prefill(q, ws, topk_indices, attn_sink, scale, out, lse, T, H, num_kv, topk, dev, s, false,
                         kv_scale);
      if (hipFreeAsync(ws, s) != hipSuccess && rc == SMLA_OK) rc = SMLA_ERR_LAUNCH;
      return rc;
    }
    (void)hipGetLastError();  // no scratch: the fp8 kernels read the codes directly
  }
  return run_prefill(q, kv, topk_indices, attn_sink, scale, out, lse, T, H, num_kv, topk, dev, s, true, kv_scale);
}

extern "C" int sparse_mla_prefill_i64(const void* q, const void* kv, const int64_t* topk_indices,
                                      const float* attn_sink, float scale, void* out, float* lse, int64_t T,
                                      int64_t H, int64_t num_kv, int64_t topk, void* stream) {
  int rc = check_args(q, kv, topk_indices, 8, attn_sink, scale, out, lse, T, H, num_kv, topk, false);
  if (rc != SMLA_OK || T == 0) return rc;
  int dev = -1;
  if ((rc = current_device(&dev)) != SMLA_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (topk == 0) return run_prefill(q, kv, nullptr, attn_sink, scale, out, lse, T, H, num_kv, topk, dev, s);
  // H <= 16 in a single pass: the 16-row kernel reads the int64 rows itself
  if (single_pass16(T, H, topk, dev))
    return run_prefill(q, kv, nullptr, attn_sink, scale, out, lse, T, H, num_kv, topk, dev, s, false, 1.f, nullptr, 0,
                       topk_indices);
  const int64_t n = T * topk;
  void* ws = nullptr;
  hipMemPool_t pool = scratch_pool(dev);
  if (pool == nullptr || hipMallocFromPoolAsync(&ws, (size_t)n * sizeof(int32_t), pool, s) != hipSuccess ||
      ws == nullptr) {
    (void)hipGetLastError();
    return SMLA_ERR_NO_MEMORY;
  }
  const int64_t want = (n + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(smla_idx64_kernel, dim3(blocks), dim3(256), 0, s, topk_indices, (int32_t*)ws, n, num_kv);
  rc = hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
  if (rc == SMLA_OK)
    rc = run_prefill(q, kv, (const int32_t*)ws, attn_sink, scale, out, lse, T, H, num_kv, topk, dev, s);
  if (hipFreeAsync(ws, s) != hipSuccess && rc == SMLA_OK) rc = SMLA_ERR_LAUNCH;
  return rc;
}

extern "C" const char* sparse_mla_status_string(int status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case SMLA_ERR_BAD_SIZE: return "invalid size (T<0, H<1, num_kv<0, topk<0, or overflow)";
    case SMLA_ERR_MISALIGNED: return "misaligned pointer (q, kv, out need 16 bytes; lse, sink and int32 topk 4; int64 topk 8)";
    case SMLA_ERR_BAD_SCALE: return "scale must be finite";
    case SMLA_ERR_NO_DEVICE: return "no usable HIP device";
    case SMLA_ERR_LAUNCH: return "kernel launch failed";
    case SMLA_ERR_NO_MEMORY: return "device scratch could not be had (int64 index conversion, backward, or the no-allocation array)";
    case SMLA_ERR_SCRATCH_LIMIT:
      return "the call's split partials need more than the no-allocation scratch holds "
             "(SPARSE_MLA_NOALLOC_SCRATCH_BYTES); use sparse_mla_prefill";
    default: return "unknown status";
  }
}

extern "C" const char* sparse_mla_kernel_name(int64_t H, int64_t topk, int kv_fp8) {
  if (H < 1 || topk < 0) return nullptr;
  return pick_variant(H, topk, kv_fp8 != 0).name;
}

extern "C" int sparse_mla_version(void) { return 102; }
