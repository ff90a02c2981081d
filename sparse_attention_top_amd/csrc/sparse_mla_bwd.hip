// Sparse MLA backward (DeepSeek-V4) for MI355X / gfx950 (CDNA4).
//
// Operation: "[Triton/Gluon] [GFX950][DSV4] Sparse MLA training backward"
// (aiter PR #4766), sections "Contract" and "Structure": from q, kv, dO, the
// forward's o and sink-inclusive lse, the top-k rows and the optional sink,
// compute dq, dkv and d_sink. With x_s = scale q . kv[r_s] over the valid
// slots s of token t, P_s = exp(x_s - lse) and delta = rowsum(o * dO):
//   dS_s = P_s (dO . kv[r_s] - delta)
//   dq   = scale sum_s dS_s kv[r_s]
//   dkv[r] = sum over slots holding r of (scale dS_s q + P_s dO), over all heads
//   d_sink = -sum_t exp(sink - lse) delta
//
// Phases (each a kernel; scratch from the library's per-device pool):
//   B1 smla_bwd_dq_kernel      one workgroup per (token, group of 16 NW heads):
//      the forward's compaction and LDS-DMA tile gather; one read of each K
//      fragment feeds the S and dP MFMAs; P and dS in fp32; dQ^T += K^T dS^T
//      from the same tile; writes dq, P and scale dS (bf16, [T][H][TP], TP =
//      top-k rounded up to 32, compacted positions), the row key and entry id
//      of every compacted position, and the sink partials. At H <= 16,
//      smla_bwd_dq16_kernel: the same on 16-row tiles, four workgroups per CU.
//   B2 smla_bwd_interm_kernel  one workgroup per token: the per-slot dkv
//      contribution interm[t][j] = [scale dS ; P]^T [q ; dO], one MFMA
//      contraction over heads (both terms side by side along K).
//   B3 a stable radix sort of (row key, entry id) and the start of
//      each row's run: the scatter inverted, so each row gathers its own
//      contributors in a fixed order (deterministic, no atomics).
//   B4 smla_bwd_dkv_chunk_kernel / smla_bwd_dkv_fix_kernel: fixed 64-entry
//      chunks of the sorted entries, one wave each, sum the interm rows of
//      each row's contributors (fp32); rows spanning chunks are finished from
//      per-chunk partials in chunk order; rows nobody references get 0.
//   B5 smla_bwd_dsink_kernel   fixed-order sum of the sink partials.


#include "smla_common.h"

namespace {

using namespace smla_host;

constexpr int kBwdMaxH = 128;  // heads handled by the interm contraction (2 x 128 rows of K)

struct BwdParams {
  const uint16_t* q;
  const uint16_t* kv;
  const uint16_t* dout;
  const uint16_t* o;
  const float* lse;
  const int32_t* topk;
  const float* sink;
  uint16_t* dq;
  uint16_t* pbuf;   // P, [T][H][TP] bf16
  uint16_t* dsbuf;  // scale dS, [T][H][TP] bf16
  uint32_t* ckey;   // [T][TP]: pool row of compacted position j, or the sentinel
  uint32_t* cval;   // [T][TP]: entry id t TP + j
  int32_t* ncount;  // [T]: compacted positions used (a multiple of 32)
  float* dsink_part;  // [T][H]: exp(sink - lse) delta
  int T;
  int H;
  int topk_n;
  int TP;
  int head_groups;
  uint32_t nkv;      // slot valid iff (uint32)idx < nkv
  uint32_t sentinel;  // row key of unused positions (== nkv)
  float scale;       // for scale dS (the dkv term scale dS q)
  float scale_log2;  // logits: scale * kv_scale * log2(e)
  float kv_scale;    // 1, or the dequant scale of a pool of fp8 code values (dP = kv_scale dO . code)
  float dq_scale;    // scale * kv_scale
};

template <int NW, int NBUF>
struct BwdSmem {
  static constexpr int kTileBytes = kBK * kRowStride;
  static constexpr int kStageBytes = NW * 16 * kRowStride;
  static constexpr int kAreaBytes = NBUF * kTileBytes > kStageBytes ? NBUF * kTileBytes : kStageBytes;
  uint8_t area[kAreaBytes];
  int32_t list[kListCap];
  __device__ __forceinline__ uint32_t tile(int b) { return lds_addr(area + b * kTileBytes); }
  __device__ __forceinline__ uint32_t stage() { return lds_addr(area); }
  __device__ __forceinline__ int32_t& wcount(int c, int w) { return ((int32_t*)area)[c * NW + w]; }
};

// Fragments of a [T, H, 512] bf16 tensor in the B-operand layout of
// S^T = K X^T: lane (g, li) holds x[t, head, 32k + 8g .. +8) (zero past H).
__device__ __forceinline__ void load_frag(bf16x8 (&f)[16], const uint16_t* x, int t, int H, int head, int g) {
  if (head < H) {
    const bf16x8* src = (const bf16x8*)(x + ((size_t)t * H + head) * kD + 8 * g);
#pragma unroll
    for (int k = 0; k < 16; ++k) f[k] = src[4 * k];
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) f[k] = bf16x8{};
  }
}

// S^T = K Q^T and dP^T = K dO^T from one read of each K fragment: four
// independent MFMA chains (two halves of 16 slots, two products).
template <int KPF>
__device__ __forceinline__ void tile_sdp(uint32_t krow, const bf16x8 (&qf)[16], const bf16x8 (&df)[16], f32x4 (&s)[2],
                                         f32x4 (&dp)[2]) {
  constexpr int KST = KPF + 1;
  f32x4 acc[2][2][1];  // [S or dP][half][1]
  u32x4 kf[KST][2];
  auto kread = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    kf[k % KST][0] = ds_read_b128<64 * k>(krow);
    kf[k % KST][1] = ds_read_b128<16 * kRowStride + 64 * k>(krow);
  };
  static_for<0, KPF>([&](auto kc) { kread(kc); });
  static_for<0, 16>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k + KPF < 16) kread(Int<k + KPF>{});
    constexpr int younger = 2 * (15 - k < KPF ? 15 - k : KPF);
    lds_wait<younger>(kf[k % KST][0], kf[k % KST][1]);
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      if constexpr (k == 0) {
        mfma_s_first(acc[0][sh][0], kf[k % KST][sh], __builtin_bit_cast(u32x4, qf[k]));
        mfma_s_first(acc[1][sh][0], kf[k % KST][sh], __builtin_bit_cast(u32x4, df[k]));
      } else {
        mfma_s(acc[0][sh][0], kf[k % KST][sh], __builtin_bit_cast(u32x4, qf[k]));
        mfma_s(acc[1][sh][0], kf[k % KST][sh], __builtin_bit_cast(u32x4, df[k]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  mfma_vgpr_drain2<1>(acc);
#pragma unroll
  for (int sh = 0; sh < 2; ++sh) {
    s[sh] = acc[0][sh][0];
    dp[sh] = acc[1][sh][0];
  }
}

// Per token, lane (g, li) of a wave: the q and dO fragments of its head,
// delta = rowsum(o . dO) of that head, its lse in log2 units, and the sink
// partial exp(sink - lse) delta (zero fragments and no partial past H).
__device__ __forceinline__ void dq_setup(const BwdParams& p, int t, int head, int g, bf16x8 (&qf)[16],
                                         bf16x8 (&df)[16], float& delta, float& lse_l2) {
  const bool hv = head < p.H;
  load_frag(qf, p.q, t, p.H, head, g);
  load_frag(df, p.dout, t, p.H, head, g);
  {
    bf16x8 of[16];
    load_frag(of, p.o, t, p.H, head, g);
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) part += (float)of[k][e] * (float)df[k][e];
    delta = row4_sum(part);  // the four 16-lane groups hold the four quarters of d
  }
  const float lse_v = hv ? p.lse[(size_t)t * p.H + head] : 0.f;
  lse_l2 = lse_v * kLog2e;
  if (p.sink != nullptr && hv && g == 0) {
    const float sk = p.sink[head];
    p.dsink_part[(size_t)t * p.H + head] = (sk == -INFINITY) ? 0.f : __expf(sk - lse_v) * delta;
  }
}

// ---- B1: dq, P, scale dS, compacted row keys, sink partials ----
template <int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1))) void smla_bwd_dq_kernel(
    const BwdParams p) {
  constexpr int AHEAD = NBUF - 1;
  __shared__ __attribute__((aligned(16))) BwdSmem<NW, NBUF> sm;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int li = lane & 15;
  const int vb = xcd_remap(blockIdx.x, gridDim.x);
  const int t = p.T - 1 - vb / p.head_groups;
  const int hg = vb % p.head_groups;
  const int head_base = (hg * NW + w) * 16;
  const int head = head_base + li;
  const bool hv = head < p.H;

  bf16x8 qf[16], df[16];
  float delta, lse_l2;
  dq_setup(p, t, head, g, qf, df, delta, lse_l2);

  f32x4 acc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 pk;

  const int32_t* trow = p.topk + (size_t)t * p.topk_n;
  const uint16_t* kvp = p.kv;
  const size_t prow = ((size_t)t * p.H + head) * p.TP;  // this lane's P / dS row
  int jbase = 0;  // compacted position of the segment's first entry (a multiple of 32)
  for (int seg0 = 0; seg0 < p.topk_n; seg0 += kListCap) {
    if (seg0 > 0 && NW > 1) lds_barrier();  // previous segment's list and tiles fully consumed
    const int n = compact_segment<NW>(trow + seg0, min(kListCap, p.topk_n - seg0), p.nkv, sm, lane, w);
    const int npos = (n + kBK - 1) / kBK * kBK;
    if (hg == 0) {
      for (int i = threadIdx.x; i < npos; i += NW * 64) {
        const size_t e = (size_t)t * p.TP + jbase + i;
        p.ckey[e] = i < n ? (uint32_t)sm.list[i] : p.sentinel;
        p.cval[e] = (uint32_t)e;
      }
    }
    const int ntiles = npos / kBK;
    if (ntiles == 0) continue;
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
      TileIssue<NW> is;
      is.init(sm.list, i, n, i < ntiles, sm.tile(i), kvp, lane, w);
      is.all(lane);
    }
    for (int j = 0; j < ntiles; ++j) {
      int after = 0;  // this wave's gather loads issued after tile j's (stores in between only add to the wait)
#pragma unroll
      for (int i = 1; i < AHEAD; ++i)
        if (j + i < ntiles) after += tile_dma<NW>(j + i, n, w);
      wait_vmcnt_le(after);
      if constexpr (NW > 1) lds_barrier();
      TileIssue<NW> is;
      is.init(sm.list, j + AHEAD, n, j + AHEAD < ntiles, sm.tile((j + AHEAD) % NBUF), kvp, lane, w);
      const uint32_t tb = sm.tile(j % NBUF);
      f32x4 s[2], dp[2];
      tile_sdp<2>(k_frag_addr(tb, g, li), qf, df, s, dp);
      const int cnt = tile_rows(j, n);
      bf16x4 pst[2], dst[2];
#pragma unroll
      for (int sh = 0; sh < 2; ++sh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = sh * 16 + 4 * g + i;
          const float pr = slot < cnt ? __builtin_amdgcn_exp2f(s[sh][i] * p.scale_log2 - lse_l2) : 0.f;
          const float ds = pr * (dp[sh][i] * p.kv_scale - delta);
          pk[sh * 4 + i] = (__bf16)ds;
          pst[sh][i] = (__bf16)pr;
          dst[sh][i] = (__bf16)(ds * p.scale);
        }
      if (hv) {
        const size_t o0 = prow + jbase + j * kBK + 4 * g;
        *(bf16x4*)(p.pbuf + o0) = pst[0];
        *(bf16x4*)(p.pbuf + o0 + 16) = pst[1];
        *(bf16x4*)(p.dsbuf + o0) = dst[0];
        *(bf16x4*)(p.dsbuf + o0 + 16) = dst[1];
      }
      is.all(lane);
      tile_pv(v_frag_addr(tb, g, li), pk, acc);  // dQ^T += K^T dS^T (V == K)
    }
    jbase += npos;
  }
  if (hg == 0) {
    for (int i = jbase + threadIdx.x; i < p.TP; i += NW * 64) {
      const size_t e = (size_t)t * p.TP + i;
      p.ckey[e] = p.sentinel;
      p.cval[e] = (uint32_t)e;
    }
    if (threadIdx.x == 0) p.ncount[t] = jbase;
  }

  // dq = scale acc, staged through LDS for whole-row stores (as the forward's o)
  if constexpr (NW > 1) lds_barrier();
  const uint32_t ob = sm.stage() + (uint32_t)w * 16 * kRowStride;
  mfma_agpr_drain(acc);
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) {
    const f32x4 v = acc[dt] * p.dq_scale;
    const bf16x4 v4 = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *(LDS_AS bf16x4*)(uintptr_t)(ob + li * kRowStride + 32 * dt + 8 * g) = v4;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int hr = head_base + r;
    const u32x4 val = *(LDS_AS const u32x4*)(uintptr_t)(ob + r * kRowStride + 16 * lane);
    if (hr < p.H) *(u32x4*)(p.dq + ((size_t)t * p.H + hr) * kD + 8 * lane) = val;
  }
}

// ---- B1 at H <= 16: 16-row tiles ----
// The same phase for one wave of up to 16 heads on 16-row tiles. A ring of two
// and 640-entry compaction segments take 36 KiB of LDS, so four workgroups
// share a CU, one wave on each SIMD, where the 32-row ring's 76 KiB leaves two
// of the four SIMDs idle (the registers allow one wave per SIMD either way).
// The next tile is gathered at the top of each iteration, under this tile's S,
// dP, stores and P.V. 640 is a multiple of 32, so segments still start on
// multiples of 32 positions and P, scale dS, the row keys and the position
// counts keep the layout the later phases read; a segment's positions are
// padded to its multiple of 32 with an all-invalid tile where needed.
constexpr int kBwd16Cap = 640;
static_assert(kBwd16Cap % kBK == 0, "segments start on multiples of 32 positions");

template <int CAP>
struct BwdSmem16 {
  static constexpr int kTileBytes = kBK16 * kRowStride;
  uint8_t area[2 * kTileBytes];  // ring of two tiles; the first 16 rows stage dq at the end
  int32_t list[CAP];
  __device__ __forceinline__ uint32_t tile(int b) { return lds_addr(area + b * kTileBytes); }
  __device__ __forceinline__ uint32_t stage() { return lds_addr(area); }
};

// S^T = K Q^T and dP^T = K dO^T for a 16-row tile from one read of each K
// fragment: s and dp hold S^T and dP^T[slot 4g + i][head li]; four MFMA chains
// (each product split by k parity).
template <int KPF>
__device__ __forceinline__ void tile_sdp16(uint32_t krow, const bf16x8 (&qf)[16], const bf16x8 (&df)[16], f32x4& s,
                                           f32x4& dp) {
  constexpr int KST = KPF + 1;
  f32x4 a[2][2];  // [S or dP][k parity]
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
    if constexpr (k < 2) {
      mfma_s_first(a[0][k], kf[k % KST], __builtin_bit_cast(u32x4, qf[k]));
      mfma_s_first(a[1][k], kf[k % KST], __builtin_bit_cast(u32x4, df[k]));
    } else {
      mfma_s(a[0][k & 1], kf[k % KST], __builtin_bit_cast(u32x4, qf[k]));
      mfma_s(a[1][k & 1], kf[k % KST], __builtin_bit_cast(u32x4, df[k]));
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // MFMA write -> VALU read distance
  asm volatile("" : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[1][0]), "+v"(a[1][1]));
  s = a[0][0] + a[0][1];
  dp = a[1][0] + a[1][1];
}

template <int CAP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1))) void smla_bwd_dq16_kernel(
    const BwdParams p) {
  __shared__ __attribute__((aligned(16))) BwdSmem16<CAP> sm;

  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int li = lane & 15;
  const int t = p.T - 1 - xcd_remap(blockIdx.x, gridDim.x);  // H <= 16: one head group per token
  const int head = li;

  bf16x8 qf[16], df[16];
  float delta, lse_l2;
  dq_setup(p, t, head, g, qf, df, delta, lse_l2);

  f32x4 acc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = p.topk + (size_t)t * p.topk_n;
  const size_t prow = ((size_t)t * p.H + head) * p.TP;  // this lane's P / dS row
  int jbase = 0;  // compacted position of the segment's first entry (a multiple of 32)
  for (int seg0 = 0; seg0 < p.topk_n; seg0 += CAP) {
    const int n = compact_segment<1, BwdSmem16<CAP>, CAP>(trow + seg0, min(CAP, p.topk_n - seg0), p.nkv, sm, lane, 0);
    const int npos = (n + kBK - 1) / kBK * kBK;
    for (int i = lane; i < npos; i += 64) {
      const size_t e = (size_t)t * p.TP + jbase + i;
      p.ckey[e] = i < n ? (uint32_t)sm.list[i] : p.sentinel;
      p.cval[e] = (uint32_t)e;
    }
    const int ntiles = npos / kBK16;  // tiles past n (at most one) are all-invalid: zero P and dS
    if (ntiles == 0) continue;
    {
      TileIssue<1, kBK16> is;
      is.init(sm.list, 0, n, true, sm.tile(0), p.kv, lane, 0);
      is.all(lane);
    }
    for (int j = 0; j < ntiles; ++j) {
      const bool next = j + 1 < ntiles;
      {
        // tile j + 1 into the slot whose last reader, P.V of tile j - 1, has completed
        TileIssue<1, kBK16> is;
        is.init(sm.list, j + 1, n, next, sm.tile((j + 1) & 1), p.kv, lane, 0);
        is.all(lane);
      }
      wait_vmcnt_le(next ? kBK16 : 0);  // tile j landed (only tile j + 1's loads may be younger)
      const uint32_t tb = sm.tile(j & 1);
      f32x4 sv, dpv;
      tile_sdp16<2>(k_frag_addr(tb, g, li), qf, df, sv, dpv);
      const int cnt = min(kBK16, n - j * kBK16);
      bf16x4 pk, pst, dst;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = 4 * g + i;
        const float pr = slot < cnt ? __builtin_amdgcn_exp2f(sv[i] * p.scale_log2 - lse_l2) : 0.f;
        const float ds = pr * (dpv[i] * p.kv_scale - delta);
        pk[i] = (__bf16)ds;
        pst[i] = (__bf16)pr;
        dst[i] = (__bf16)(ds * p.scale);
      }
      if (head < p.H) {
        const size_t o0 = prow + jbase + j * kBK16 + 4 * g;
        *(bf16x4*)(p.pbuf + o0) = pst;
        *(bf16x4*)(p.dsbuf + o0) = dst;
      }
      tile_pv16(v_frag_addr(tb, g, li), pk, acc);  // dQ^T += K^T dS^T (V == K)
    }
    jbase += npos;
  }
  for (int i = jbase + lane; i < p.TP; i += 64) {
    const size_t e = (size_t)t * p.TP + i;
    p.ckey[e] = p.sentinel;
    p.cval[e] = (uint32_t)e;
  }
  if (lane == 0) p.ncount[t] = jbase;

  // dq = scale acc, staged through LDS for whole-row stores (no tile load is
  // in flight: the last tile issued none, and every earlier one was waited for)
  const uint32_t ob = sm.stage();
  mfma_agpr_drain(acc);
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) {
    const f32x4 v = acc[dt] * p.dq_scale;
    const bf16x4 v4 = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *(LDS_AS bf16x4*)(uintptr_t)(ob + li * kRowStride + 32 * dt + 8 * g) = v4;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const u32x4 val = *(LDS_AS const u32x4*)(uintptr_t)(ob + r * kRowStride + 16 * lane);
    if (r < p.H) *(u32x4*)(p.dq + ((size_t)t * p.H + r) * kD + 8 * lane) = val;
  }
}

// ---- B2: interm[t][j][d] = sum_h scale dS[t][h][j] q[t][h][d] + P[t][h][j] dO[t][h][d] ----
// One workgroup of 8 waves per token; wave w owns the 64 columns d = 64 w ..
// 64 w + 63 (four 16-column d-tiles). C^T[d][j] = X^T[d][k] Y[k][j], k running
// over the 2 Hp rows of X = [q ; dO] and of Y = [scale dS ; P] (Hp = H rounded
// up to 16; rows of padded heads are zero), KS = 2 Hp / 32 MFMA k-steps. A wave's
// X^T fragments (4 KS of them) do not depend on j: they are read once per token,
// from [q ; dO] staged a quarter of d (128 columns) at a time, and stay in
// registers. Y is staged per 32-position tile (double-buffered, the next tile's
// LDS-DMA in flight during the current one). Both operands come from
// transposing LDS reads that give lane (g, li) rows k0 + 4g .. +3 and
// k0 + 16 + 4g .. +3 at one column, the same rows for both, so the K order
// matches.
struct InterParams {
  const uint16_t* q;
  const uint16_t* dout;
  const uint16_t* pbuf;
  const uint16_t* dsbuf;
  const int32_t* ncount;
  uint16_t* interm;  // [T][TP][512]
  int T;
  int H;
  int Hp;
  int TP;
};

// LDS of the interm kernel, sized for its 32 KS rows of [q ; dO] and [scale dS ; P],
// and the staging of one 32-position output tile (32 rows of kRowStride) for
// whole-row stores: in the [q ; dO] buffers once the fragments are read, or in
// an area of its own when those are smaller.
template <bool OWN>
struct InterStage {  // the staging area of its own
  uint8_t o[kBK * kRowStride];
  __device__ __forceinline__ const void* own() const { return o; }
};
template <>
struct InterStage<false> {  // empty: the staging reuses the [q ; dO] buffers
  __device__ __forceinline__ const void* own() const { return nullptr; }
};
template <int KS>
struct InterSmem : InterStage<(2 * 32 * KS * 256 < kBK * kRowStride)> {
  static constexpr bool kOwnStage = 2 * 32 * KS * 256 < kBK * kRowStride;
  uint8_t x[2][32 * KS][256];  // [q ; dO] rows, 128 columns of d, double-buffered
  uint8_t y[2][32 * KS][64];   // [scale dS ; P] rows of a 32-position tile, double-buffered
  __device__ __forceinline__ uint32_t stage() { return lds_addr(kOwnStage ? this->own() : &x[0][0][0]); }
};

// Stage quarter qd of [q ; dO] (columns 128 qd ..): row k = 4i + L/16, bytes 16 (L % 16); wave w issues i = w, w + 8, ...
__device__ __forceinline__ void interm_stage_x(const InterParams& p, uint8_t (*x)[256], int t, int qd, int lane, int w) {
  const int rows = 2 * p.Hp;
  const uint16_t* zero = uniform_ptr(kZeroRowBf16);
  for (int i = w; i * 4 < rows; i += 8) {
    const int k = 4 * i + (lane >> 4);
    const int h = k < p.Hp ? k : k - p.Hp;
    const uint16_t* base = k < p.Hp ? p.q : p.dout;
    const uint16_t* src =
        h < p.H ? base + ((size_t)t * p.H + h) * kD + 128 * qd + 8 * (lane & 15) : zero + 8 * (lane & 15);
    __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)(uintptr_t)lds_addr(&x[4 * i][0]), 16, 0, 0);
  }
}
// Stage tile jt of [scale dS ; P]: row k = 16i + L/4, bytes 16 (L % 4).
__device__ __forceinline__ void interm_stage_y(const InterParams& p, uint8_t (*y)[64], int t, int jt, int lane, int w) {
  const int rows = 2 * p.Hp;
  const uint16_t* zero = uniform_ptr(kZeroRowBf16);
  for (int i = w; i * 16 < rows; i += 8) {
    const int k = 16 * i + (lane >> 2);
    const int h = k < p.Hp ? k : k - p.Hp;
    const uint16_t* base = k < p.Hp ? p.dsbuf : p.pbuf;
    const uint16_t* src = h < p.H ? base + ((size_t)t * p.H + h) * p.TP + jt * kBK + 8 * (lane & 3) : zero + 8 * (lane & 3);
    __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)(uintptr_t)lds_addr(&y[16 * i][0]), 16, 0, 0);
  }
}

template <int KS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void smla_bwd_interm_kernel(
    const InterParams p) {
  __shared__ __attribute__((aligned(16))) InterSmem<KS> sm;
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int li = lane & 15;
  const int ntl = p.ncount[t] / kBK;
  if (ntl == 0) return;

  interm_stage_y(p, sm.y[0], t, 0, lane, w);
  interm_stage_x(p, sm.x[0], t, 0, lane, w);
  // lane's row in a 32-row k step (4g + li/4, and + 16) and its 8-byte column chunk
  const uint32_t lrow = (uint32_t)(4 * g + (li >> 2));
  u32x4 af[KS][4];
  static_for<0, 4>([&](auto qc) {
    constexpr int qd = decltype(qc)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // quarter qd (and Y tile 0) landed, this wave's part
    lds_barrier();                                      // ... every wave's; quarter qd - 1 no longer read
    if constexpr (qd + 1 < 4) interm_stage_x(p, sm.x[(qd + 1) & 1], t, qd + 1, lane, w);
    if (w / 2 == qd) {
      const uint32_t xb = opaque(lds_addr(&sm.x[qd & 1][0][0]) + lrow * 256 + 128 * (w & 1) + 8 * (li & 3));
      static_for<0, KS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        static_for<0, 4>([&](auto dc) {
          constexpr int dt = decltype(dc)::value;
          u32x2 a0 = ds_read_tr16_b64<ks * 32 * 256 + 32 * dt>(xb);
          u32x2 a1 = ds_read_tr16_b64<ks * 32 * 256 + 16 * 256 + 32 * dt>(xb);
          lds_wait<0>(a0, a1);
          af[ks][dt] = u32x4{a0[0], a0[1], a1[0], a1[1]};
        });
      });
    }
  });
  lds_barrier();  // every wave holds its fragments: the [q ; dO] buffers may now take the output staging

  for (int it = 0; it < ntl; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntl) interm_stage_y(p, sm.y[buf ^ 1], t, it + 1, lane, w);
    const uint32_t yb = opaque(lds_addr(&sm.y[buf][0][0]) + lrow * 64 + 8 * (li & 3));
    f32x4 c[4][2];
    u32x2 bf[2][2][2];  // [k-step parity][jt][half]
    auto bread = [&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      static_for<0, 2>([&](auto jc) {
        constexpr int jt = decltype(jc)::value;
        bf[ks & 1][jt][0] = ds_read_tr16_b64<ks * 32 * 64 + 32 * jt>(yb);
        bf[ks & 1][jt][1] = ds_read_tr16_b64<ks * 32 * 64 + 16 * 64 + 32 * jt>(yb);
      });
    };
    bread(Int<0>{});
    static_for<0, KS>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      if constexpr (ks + 1 < KS) bread(Int<ks + 1>{});
      constexpr int younger = ks + 1 < KS ? 4 : 0;
      asm volatile("s_waitcnt lgkmcnt(%4)"
                   : "+v"(bf[ks & 1][0][0]), "+v"(bf[ks & 1][0][1]), "+v"(bf[ks & 1][1][0]), "+v"(bf[ks & 1][1][1])
                   : "n"(younger));
      static_for<0, 2>([&](auto jc) {
        constexpr int jt = decltype(jc)::value;
        const u32x4 b = u32x4{bf[ks & 1][jt][0][0], bf[ks & 1][jt][0][1], bf[ks & 1][jt][1][0], bf[ks & 1][jt][1][1]};
        static_for<0, 4>([&](auto dc) {
          constexpr int dt = decltype(dc)::value;
          if constexpr (ks == 0) mfma_s_first(c[dt][jt], af[ks][dt], b);
          else mfma_s(c[dt][jt], af[ks][dt], b);
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // MFMA write -> VALU read distance
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) asm volatile("" : "+v"(c[dt][jt]));
    // lane holds C^T[d = 64 w + 16 dt + 4 g + i][j = 16 jt + li] of this tile: staged as rows j
    const uint32_t ob = sm.stage();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *(LDS_AS bf16x4*)(uintptr_t)(ob + (16 * jt + li) * kRowStride + 2 * (64 * w + 16 * dt + 4 * g)) =
            bf16x4{(__bf16)c[dt][jt][0], (__bf16)c[dt][jt][1], (__bf16)c[dt][jt][2], (__bf16)c[dt][jt][3]};
    lds_barrier();  // the tile is staged; no wave reads this Y tile any more
    // wave w stores rows 4 w .. 4 w + 3, one whole 1 KiB row per instruction
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * w + r;
      const u32x4 v = *(LDS_AS const u32x4*)(uintptr_t)(ob + j * kRowStride + 16 * lane);
      *(u32x4*)(p.interm + ((size_t)t * p.TP + it * kBK + j) * kD + 8 * lane) = v;
    }
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // the next tile's rows landed (only the 4 stores may be younger)
    lds_barrier();                                     // ... every wave's; the staging is free again
  }
}

// ---- B3: stable LSD radix sort of (row key, entry id), 8-bit digits ----
// Each pass is a stable counting sort on one digit of the key: blocks of
// kSortBlock pairs count their digits (count), one workgroup per digit turns
// that digit's block counts into exclusive offsets and a total (scan), and each block
// places its pairs in order (scatter): within a chunk of 256 pairs, the lanes
// of a wave holding the same digit are found with one ballot per digit bit,
// ranked by lane, and offset by the same digit's count in the lower waves of
// the chunk and in the block's earlier chunks. Every rank is a count, never
// the order of an atomic, so the result is the same on every call. No memory
// is set beforehand: each pass writes every count it reads.
constexpr int kSortItems = 16;                 // chunks of 256 pairs per block
constexpr int kSortBlock = 256 * kSortItems;   // pairs per block

__global__ __launch_bounds__(256) void smla_sort_count_kernel(const uint32_t* __restrict__ keys, uint32_t n,
                                                              int shift, uint32_t* __restrict__ counts) {
  __shared__ uint32_t hist[256];
  hist[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t base = blockIdx.x * (uint32_t)kSortBlock;
#pragma unroll 4
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t e = base + i * 256 + threadIdx.x;
    if (e < n) atomicAdd(&hist[(keys[e] >> shift) & 255u], 1u);
  }
  __syncthreads();
  counts[threadIdx.x * gridDim.x + blockIdx.x] = hist[threadIdx.x];
}

// Exclusive prefix sum over the blocks of one digit's counts (counts[d nb ..
// d nb + nb), one workgroup per digit d), in tiles of 1024 (four per thread,
// contiguous); the digit's total goes to totals[d].
__global__ __launch_bounds__(256) void smla_sort_scan_kernel(uint32_t* __restrict__ counts, uint32_t nb,
                                                             uint32_t* __restrict__ totals) {
  __shared__ uint32_t part[256];
  uint32_t* c = counts + (size_t)blockIdx.x * nb;
  uint32_t carry = 0;
  for (uint32_t t0 = 0; t0 < nb; t0 += 1024) {
    uint32_t v[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t i = t0 + 4 * threadIdx.x + k;
      v[k] = i < nb ? c[i] : 0u;
      sum += v[k];
    }
    part[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const uint32_t x = threadIdx.x >= (uint32_t)off ? part[threadIdx.x - off] : 0u;
      __syncthreads();
      part[threadIdx.x] += x;
      __syncthreads();
    }
    uint32_t run = carry + (threadIdx.x ? part[threadIdx.x - 1] : 0u);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t i = t0 + 4 * threadIdx.x + k;
      if (i < nb) c[i] = run;
      run += v[k];
    }
    carry += part[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

__global__ __launch_bounds__(256) void smla_sort_scatter_kernel(const uint32_t* __restrict__ kin,
                                                                const uint32_t* __restrict__ vin,
                                                                uint32_t* __restrict__ kout, uint32_t* __restrict__ vout,
                                                                uint32_t n, int shift,
                                                                const uint32_t* __restrict__ offs,
                                                                const uint32_t* __restrict__ totals) {
  __shared__ uint32_t run[256];      // per digit: where this block's next pair of that digit goes
  __shared__ uint32_t wcnt[4][256];  // per wave and digit: pairs of that digit in the current chunk
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // the digit's start: the totals of the lower digits (an exclusive scan of 256 in LDS)
  run[threadIdx.x] = totals[threadIdx.x];
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t x = threadIdx.x >= (uint32_t)off ? run[threadIdx.x - off] : 0u;
    __syncthreads();
    run[threadIdx.x] += x;
    __syncthreads();
  }
  const uint32_t start = run[threadIdx.x] - totals[threadIdx.x];
  __syncthreads();
  run[threadIdx.x] = start + offs[threadIdx.x * gridDim.x + blockIdx.x];
#pragma unroll
  for (int k = 0; k < 4; ++k) wcnt[k][threadIdx.x] = 0u;
  __syncthreads();
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;  // lanes lower than this one
  const uint32_t base = blockIdx.x * (uint32_t)kSortBlock;
  uint32_t keys[kSortItems], vals[kSortItems];  // all of this thread's pairs first: one load latency per block
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t e = base + i * 256 + threadIdx.x;
    keys[i] = e < n ? kin[e] : 0u;
    vals[i] = e < n ? vin[e] : 0u;
  }
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t e = base + i * 256 + threadIdx.x;
    const bool act = e < n;
    const uint32_t key = keys[i];
    const uint32_t val = vals[i];
    const uint32_t d = (key >> shift) & 255u;
    uint64_t peers = __ballot(act);  // active lanes of this wave with the same digit
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t ones = __ballot((d >> bit) & 1u);
      peers &= ((d >> bit) & 1u) ? ones : ~ones;
    }
    const uint32_t rank = (uint32_t)__popcll(peers & below);
    if (act && rank == 0) wcnt[w][d] = (uint32_t)__popcll(peers);
    __syncthreads();
    if (act) {
      uint32_t pos = run[d] + rank;
      for (int k = 0; k < w; ++k) pos += wcnt[k][d];
      kout[pos] = key;
      vout[pos] = val;
    }
    __syncthreads();
    run[threadIdx.x] += wcnt[0][threadIdx.x] + wcnt[1][threadIdx.x] + wcnt[2][threadIdx.x] + wcnt[3][threadIdx.x];
#pragma unroll
    for (int k = 0; k < 4; ++k) wcnt[k][threadIdx.x] = 0u;
    __syncthreads();
  }
}

// ---- B3: start of each row's run in the sorted keys (lower bound) ----
__global__ __launch_bounds__(256) void smla_bwd_rowstart_kernel(const uint32_t* __restrict__ skey, uint32_t n,
                                                                uint32_t nrows, uint32_t* __restrict__ row_start) {
  const uint32_t r = blockIdx.x * 256 + threadIdx.x;
  if (r > nrows) return;
  uint32_t lo = 0, hi = n;
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo) / 2;
    if (skey[mid] < r) lo = mid + 1;
    else hi = mid;
  }
  row_start[r] = lo;
}

// ---- B4: dkv[r] = sum of the interm rows of r's contributors (fp32), bf16 ----
// The sorted entries are cut into chunks of kChunk; one wave per chunk sums
// each run of equal keys inside it (lane L: d = 8L .. 8L+7). A run that is a
// whole row is stored to dkv at once; the run at a chunk's start that belongs
// to a row begun in an earlier chunk goes to head[chunk], the run at its end
// that continues past it to tail[chunk] (fp32). B4b then finishes every row
// that spans chunks c0 .. c1 as tail[c0] + head[c0 + 1] + ... + head[c1], in
// that order, and zero-fills rows no slot holds. The order of every sum is
// fixed by the sort, so dkv is deterministic.
// With token passes (acc != NULL), each pass adds its row sums to an fp32
// accumulator instead (every row is touched by one wave per pass, passes run in
// token order), and smla_bwd_dkv_out_kernel rounds it to bf16 at the end.
constexpr int kChunk = 64;

__device__ __forceinline__ void dkv_flush(const float (&a)[8], uint32_t r, uint32_t s0, uint32_t s1,
                                          const uint32_t* __restrict__ row_start, uint16_t* __restrict__ dkv,
                                          float* __restrict__ acc, float* __restrict__ head, float* __restrict__ tail,
                                          uint32_t c, int lane) {
  const bool before = row_start[r] < s0;
  const bool after = row_start[r + 1] > s1;
  if (!before && !after) {
    if (acc != nullptr) {
      f32x4* dst = (f32x4*)(acc + (size_t)r * kD + 8 * lane);
      dst[0] += f32x4{a[0], a[1], a[2], a[3]};
      dst[1] += f32x4{a[4], a[5], a[6], a[7]};
      return;
    }
    *(bf16x8*)(dkv + (size_t)r * kD + 8 * lane) = bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                                                         (__bf16)a[4], (__bf16)a[5], (__bf16)a[6], (__bf16)a[7]};
  } else {
    float* dst = (before ? head : tail) + (size_t)c * kD + 8 * lane;
    *(f32x4*)dst = f32x4{a[0], a[1], a[2], a[3]};
    *(f32x4*)(dst + 4) = f32x4{a[4], a[5], a[6], a[7]};
  }
}

__global__ __launch_bounds__(256) void smla_bwd_dkv_chunk_kernel(const uint32_t* __restrict__ skey,
                                                                 const uint32_t* __restrict__ sval,
                                                                 const uint32_t* __restrict__ row_start,
                                                                 const uint16_t* __restrict__ interm,
                                                                 uint16_t* __restrict__ dkv, float* __restrict__ acc,
                                                                 float* __restrict__ head, float* __restrict__ tail,
                                                                 uint32_t num_kv) {
  const int lane = threadIdx.x & 63;
  const uint32_t c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint32_t nv = row_start[num_kv];  // entries with a valid key
  const uint32_t e0 = c * kChunk;
  if (e0 >= nv) return;
  const uint32_t e1 = min(e0 + (uint32_t)kChunk, nv);
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  uint32_t cur = skey[e0], seg = e0;
  for (uint32_t e = e0; e < e1; e += 4) {
    u32x4 x[4];
    uint32_t rk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t ee = e + u < e1 ? e + u : e1 - 1;  // in range; the extra loads are not used
      rk[u] = skey[ee];
      x[u] = *(const u32x4*)(interm + (size_t)sval[ee] * kD + 8 * lane);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (e + u >= e1) break;
      if (rk[u] != cur) {
        dkv_flush(a, cur, seg, e + u, row_start, dkv, acc, head, tail, c, lane);
        cur = rk[u];
        seg = e + u;
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = 0.f;
      }
      const bf16x8 v = __builtin_bit_cast(bf16x8, x[u]);
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] += (float)v[i];
    }
  }
  dkv_flush(a, cur, seg, e1, row_start, dkv, acc, head, tail, c, lane);
}

__global__ __launch_bounds__(256) void smla_bwd_dkv_fix_kernel(const uint32_t* __restrict__ row_start,
                                                               const float* __restrict__ head,
                                                               const float* __restrict__ tail, uint16_t* __restrict__ dkv,
                                                               float* __restrict__ acc, int64_t num_kv) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= num_kv) return;
  const uint32_t s0 = row_start[r], s1 = row_start[r + 1];
  uint16_t* dst = dkv + r * kD + 8 * lane;
  if (s0 == s1) {
    if (acc == nullptr) *(u32x4*)dst = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const uint32_t c0 = s0 / kChunk, c1 = (s1 - 1) / kChunk;
  if (c0 == c1) return;  // the chunk pass stored it
  f32x4 lo = *(const f32x4*)(tail + (size_t)c0 * kD + 8 * lane);
  f32x4 hi = *(const f32x4*)(tail + (size_t)c0 * kD + 8 * lane + 4);
  for (uint32_t c = c0 + 1; c <= c1; ++c) {
    lo += *(const f32x4*)(head + (size_t)c * kD + 8 * lane);
    hi += *(const f32x4*)(head + (size_t)c * kD + 8 * lane + 4);
  }
  if (acc != nullptr) {
    f32x4* a = (f32x4*)(acc + r * kD + 8 * lane);
    a[0] += lo;
    a[1] += hi;
    return;
  }
  *(bf16x8*)dst = bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                         (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
}

// dkv = bf16(acc), after the last token pass
__global__ __launch_bounds__(256) void smla_bwd_dkv_out_kernel(const float* __restrict__ acc,
                                                              uint16_t* __restrict__ dkv, int64_t num_kv) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= num_kv) return;
  const f32x4 lo = *(const f32x4*)(acc + r * kD + 8 * lane);
  const f32x4 hi = *(const f32x4*)(acc + r * kD + 8 * lane + 4);
  *(bf16x8*)(dkv + r * kD + 8 * lane) = bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                                              (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
}

// ---- B5: d_sink[h] = -sum_t part[t][h], in a fixed order ----
__global__ __launch_bounds__(256) void smla_bwd_dsink_kernel(const float* __restrict__ part, int T, int H,
                                                             float* __restrict__ d_sink) {
  __shared__ float red[256];
  const int h = blockIdx.x;
  float acc = 0.f;
  for (int t = threadIdx.x; t < T; t += 256) acc += part[(size_t)t * H + h];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) d_sink[h] = -red[0];
}

// Zero fill (rows of dkv when nothing is gathered; d_sink without tokens).
__global__ __launch_bounds__(256) void smla_zero_kernel(uint32_t* __restrict__ p, int64_t n_words) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_words; i += stride) p[i] = 0u;
}

int bwd_nw(int64_t H) { return H <= 16 ? 1 : (H <= 32 ? 2 : 4); }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Count buffer of the radix sort for n pairs: 256 digits per block, then the 256 digit totals.
size_t sort_count_bytes(int64_t n) { return (size_t)256 * (size_t)((n + kSortBlock - 1) / kSortBlock + 1) * 4; }

// Sort n (key, value) pairs by the low end_bit bits of the key, stably: the
// pairs move between (k0, v0) and (k1, v1) once per 8-bit digit; the sorted
// pairs end in (k0, v0) after an even number of passes, else in (k1, v1)
// (*in_first says which).
hipError_t sort_pairs(uint32_t* k0, uint32_t* v0, uint32_t* k1, uint32_t* v1, uint32_t* counts, int64_t n,
                      int end_bit, hipStream_t s, bool* in_first) {
  const unsigned nb = (unsigned)((n + kSortBlock - 1) / kSortBlock);
  bool first = true;
  for (int shift = 0; shift < end_bit && n > 0; shift += 8) {
    const uint32_t* kin = first ? k0 : k1;
    const uint32_t* vin = first ? v0 : v1;
    uint32_t* kout = first ? k1 : k0;
    uint32_t* vout = first ? v1 : v0;
    hipLaunchKernelGGL(smla_sort_count_kernel, dim3(nb), dim3(256), 0, s, kin, (uint32_t)n, shift, counts);
    hipLaunchKernelGGL(smla_sort_scan_kernel, dim3(256), dim3(256), 0, s, counts, nb, counts + (size_t)256 * nb);
    hipLaunchKernelGGL(smla_sort_scatter_kernel, dim3(nb), dim3(256), 0, s, kin, vin, kout, vout, (uint32_t)n, shift,
                       (const uint32_t*)counts, (const uint32_t*)(counts + (size_t)256 * nb));
    first = !first;
  }
  *in_first = first;
  return hipGetLastError();
}

// Scratch of one token pass, at most (unless one token alone needs more): the
// passes are chosen so that T_pass * per-token bytes stays below it.
constexpr size_t kBwdPassBytes = (size_t)4 << 30;

// Argument checks of the backward (no device access); idx_align: 4 for int32
// rows, 8 for int64.
int bwd_check(const void* q, const void* kv, const void* dout, const void* o, const float* lse,
              const void* topk_indices, size_t idx_align, const float* attn_sink, float scale, void* dq, void* dkv,
              float* d_sink, int64_t T, int64_t H, int64_t num_kv, int64_t topk, int64_t chunk_tokens) {
  if (T < 0 || H < 1 || num_kv < 0 || topk < 0 || chunk_tokens < 0) return SMLA_ERR_BAD_SIZE;
  if (H > kBwdMaxH || T > INT32_MAX || topk > INT32_MAX || num_kv >= ((int64_t)1 << 31)) return SMLA_ERR_BAD_SIZE;
  if (!isfinite(scale)) return SMLA_ERR_BAD_SCALE;
  const int64_t TP = (topk + kBK - 1) / kBK * kBK;
  if (T * TP >= ((int64_t)1 << 31)) return SMLA_ERR_BAD_SIZE;
  if (T > 0 && (!q || !dout || !o || !lse || !dq)) return SMLA_ERR_NULL_POINTER;
  if (T > 0 && topk > 0 && !topk_indices) return SMLA_ERR_NULL_POINTER;
  if (num_kv > 0 && (!kv || !dkv)) return SMLA_ERR_NULL_POINTER;
  if (attn_sink && !d_sink) return SMLA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(dout, 16) || !aligned(o, 16) || !aligned(dq, 16) || (kv && !aligned(kv, 16)) ||
      (dkv && !aligned(dkv, 16)))
    return SMLA_ERR_MISALIGNED;
  if (!aligned(lse, 4) || (topk_indices && !aligned(topk_indices, idx_align)) || (attn_sink && !aligned(attn_sink, 4)) ||
      (d_sink && !aligned(d_sink, 4)))
    return SMLA_ERR_MISALIGNED;
  return SMLA_OK;
}

int run_backward(const void* q, const void* kv, const void* dout, const void* o, const float* lse,
                 const int32_t* topk_indices, const float* attn_sink, float scale, void* dq, void* dkv, float* d_sink,
                 int64_t T, int64_t H, int64_t num_kv, int64_t topk, int64_t chunk_tokens, void* stream,
                 float kv_scale = 1.f) {
  const int rc0 = bwd_check(q, kv, dout, o, lse, topk_indices, 4, attn_sink, scale, dq, dkv, d_sink, T, H, num_kv,
                            topk, chunk_tokens);
  if (rc0 != SMLA_OK) return rc0;
  const int64_t TP = (topk + kBK - 1) / kBK * kBK;
  int dev = 0;
  if (current_device(&dev) != SMLA_OK) return SMLA_ERR_NO_DEVICE;
  hipStream_t s = (hipStream_t)stream;

  if (T == 0 || TP == 0) {
    // No slot at all: every gradient is zero (with a sink, each token's o is 0,
    // so delta and the sink gradient are 0 too).
    if (num_kv > 0) hipLaunchKernelGGL(smla_zero_kernel, dim3(1024), dim3(256), 0, s, (uint32_t*)dkv, num_kv * kD / 2);
    if (T > 0) hipLaunchKernelGGL(smla_zero_kernel, dim3(1024), dim3(256), 0, s, (uint32_t*)dq, T * H * kD / 2);
    if (attn_sink) hipLaunchKernelGGL(smla_zero_kernel, dim3(1), dim3(256), 0, s, (uint32_t*)d_sink, H);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
  }

  const int nw = bwd_nw(H);
  const int64_t heads_per_wg = 16 * nw;
  const int64_t head_groups = (H + heads_per_wg - 1) / heads_per_wg;
  const int Hp = (int)((H + 15) / 16 * 16);

  // Token passes: P, scale dS, the sort keys and the interm rows exist for one
  // pass at a time (about TP (4 H + 1104) bytes per token). With more than one
  // pass, each adds its dkv row sums to an fp32 accumulator.
  const size_t per_token = (size_t)TP * (4 * (size_t)H + 4 * 4 + 2 * kD) + 4 + (size_t)TP / kChunk * 2 * kD * 4 + 2 * kD * 4;
  int64_t C = chunk_tokens;
  if (C == 0) {  // as few passes as the bound allows, of equal size
    const int64_t cap = (int64_t)(kBwdPassBytes / per_token) > 0 ? (int64_t)(kBwdPassBytes / per_token) : 1;
    const int64_t npass = (T + cap - 1) / cap;
    C = (T + npass - 1) / npass;
  }
  C = C < 1 ? 1 : (C > T ? T : C);
  const bool passes = C < T;
  const int64_t Nc = C * TP;  // sorted entries of one pass

  const uint32_t nkv = kv ? (uint32_t)num_kv : 0u;
  int end_bit = 1;  // the sort looks at the bits the keys use (rows < nkv, the sentinel nkv)
  while (end_bit < 32 && ((uint64_t)1 << end_bit) <= (uint64_t)nkv) ++end_bit;

  // scratch layout: one pass's buffers, then what lives across passes
  const size_t sort_bytes = sort_count_bytes(Nc);
  const size_t A = 256;
  size_t off = 0;
  const size_t o_p = off;      off = align_up(off + (size_t)C * H * TP * 2, A);
  const size_t o_ds = off;     off = align_up(off + (size_t)C * H * TP * 2, A);
  const size_t o_ck = off;     off = align_up(off + (size_t)Nc * 4, A);
  const size_t o_cv = off;     off = align_up(off + (size_t)Nc * 4, A);
  const size_t o_sk = off;     off = align_up(off + (size_t)Nc * 4, A);
  const size_t o_sv = off;     off = align_up(off + (size_t)Nc * 4, A);
  const size_t o_nc = off;     off = align_up(off + (size_t)C * 4, A);
  const size_t o_it = off;     off = align_up(off + (size_t)Nc * kD * 2, A);
  const size_t nch = (size_t)(Nc + kChunk - 1) / kChunk;
  const size_t o_hd = off;     off = align_up(off + nch * kD * 4, A);
  const size_t o_tl = off;     off = align_up(off + nch * kD * 4, A);
  const size_t o_tmp = off;    off = align_up(off + sort_bytes, A);
  const size_t o_dsp = off;    off = align_up(off + (size_t)T * H * 4, A);
  const size_t o_rs = off;     off = align_up(off + (size_t)(num_kv + 1) * 4, A);
  const size_t o_acc = off;    off = align_up(off + (passes ? (size_t)num_kv * kD * 4 : 0), A);
  void* ws = nullptr;
  hipMemPool_t pool = scratch_pool(dev);
  if (pool == nullptr || hipMallocFromPoolAsync(&ws, off, pool, s) != hipSuccess || ws == nullptr) {
    (void)hipGetLastError();
    return SMLA_ERR_NO_MEMORY;
  }
  char* b = (char*)ws;
  float* acc = passes ? (float*)(b + o_acc) : nullptr;
  hipError_t err = hipSuccess;
  if (acc != nullptr && num_kv > 0) {
    hipLaunchKernelGGL(smla_zero_kernel, dim3(1024), dim3(256), 0, s, (uint32_t*)acc, num_kv * kD);
    err = hipGetLastError();
  }

  for (int64_t t0 = 0; t0 < T && err == hipSuccess; t0 += C) {
    const int64_t Tc = T - t0 < C ? T - t0 : C;  // tokens of this pass
    const int64_t Nt = Tc * TP;
    const size_t qoff = (size_t)t0 * H * kD;
    BwdParams bp;
    bp.q = (const uint16_t*)q + qoff;
    bp.kv = (const uint16_t*)kv;
    bp.dout = (const uint16_t*)dout + qoff;
    bp.o = (const uint16_t*)o + qoff;
    bp.lse = lse + (size_t)t0 * H;
    bp.topk = topk_indices ? topk_indices + (size_t)t0 * topk : nullptr;
    bp.sink = attn_sink;
    bp.dq = (uint16_t*)dq + qoff;
    bp.pbuf = (uint16_t*)(b + o_p);
    bp.dsbuf = (uint16_t*)(b + o_ds);
    bp.ckey = (uint32_t*)(b + o_ck);
    bp.cval = (uint32_t*)(b + o_cv);
    bp.ncount = (int32_t*)(b + o_nc);
    bp.dsink_part = (float*)(b + o_dsp) + (size_t)t0 * H;
    bp.T = (int)Tc;
    bp.H = (int)H;
    bp.topk_n = (int)topk;
    bp.TP = (int)TP;
    bp.head_groups = (int)head_groups;
    bp.nkv = nkv;
    bp.sentinel = nkv;
    bp.scale = scale;
    bp.scale_log2 = scale * kv_scale * kLog2e;
    bp.kv_scale = kv_scale;
    bp.dq_scale = scale * kv_scale;

    const unsigned g1 = (unsigned)(Tc * head_groups);
    if (nw == 1) hipLaunchKernelGGL((smla_bwd_dq16_kernel<kBwd16Cap>), dim3(g1), dim3(64), 0, s, bp);
    else if (nw == 2) hipLaunchKernelGGL((smla_bwd_dq_kernel<2, 2>), dim3(g1), dim3(128), 0, s, bp);
    else hipLaunchKernelGGL((smla_bwd_dq_kernel<4, 2>), dim3(g1), dim3(256), 0, s, bp);
    err = hipGetLastError();

    if (err == hipSuccess) {
      InterParams ip;
      ip.q = bp.q;
      ip.dout = bp.dout;
      ip.pbuf = bp.pbuf;
      ip.dsbuf = bp.dsbuf;
      ip.ncount = bp.ncount;
      ip.interm = (uint16_t*)(b + o_it);
      ip.T = (int)Tc;
      ip.H = (int)H;
      ip.Hp = Hp;
      ip.TP = (int)TP;
      const dim3 grid((unsigned)Tc);
      switch (Hp / 16) {
        case 1: hipLaunchKernelGGL(smla_bwd_interm_kernel<1>, grid, dim3(512), 0, s, ip); break;
        case 2: hipLaunchKernelGGL(smla_bwd_interm_kernel<2>, grid, dim3(512), 0, s, ip); break;
        case 3: hipLaunchKernelGGL(smla_bwd_interm_kernel<3>, grid, dim3(512), 0, s, ip); break;
        case 4: hipLaunchKernelGGL(smla_bwd_interm_kernel<4>, grid, dim3(512), 0, s, ip); break;
        case 5: hipLaunchKernelGGL(smla_bwd_interm_kernel<5>, grid, dim3(512), 0, s, ip); break;
        case 6: hipLaunchKernelGGL(smla_bwd_interm_kernel<6>, grid, dim3(512), 0, s, ip); break;
        case 7: hipLaunchKernelGGL(smla_bwd_interm_kernel<7>, grid, dim3(512), 0, s, ip); break;
        default: hipLaunchKernelGGL(smla_bwd_interm_kernel<8>, grid, dim3(512), 0, s, ip); break;
      }
      err = hipGetLastError();
    }
    uint32_t* skey = bp.ckey;  // where the sorted pairs end
    uint32_t* sval = bp.cval;
    if (err == hipSuccess && num_kv > 0) {
      bool in_first = true;
      err = sort_pairs(bp.ckey, bp.cval, (uint32_t*)(b + o_sk), (uint32_t*)(b + o_sv), (uint32_t*)(b + o_tmp), Nt,
                       end_bit, s, &in_first);
      skey = in_first ? bp.ckey : (uint32_t*)(b + o_sk);
      sval = in_first ? bp.cval : (uint32_t*)(b + o_sv);
    }
    if (err == hipSuccess && num_kv > 0) {
      const size_t nch_t = (size_t)(Nt + kChunk - 1) / kChunk;
      hipLaunchKernelGGL(smla_bwd_rowstart_kernel, dim3((unsigned)((num_kv + 1 + 255) / 256)), dim3(256), 0, s,
                         (const uint32_t*)skey, (uint32_t)Nt, (uint32_t)num_kv, (uint32_t*)(b + o_rs));
      hipLaunchKernelGGL(smla_bwd_dkv_chunk_kernel, dim3((unsigned)((nch_t + 3) / 4)), dim3(256), 0, s,
                         (const uint32_t*)skey, (const uint32_t*)sval, (const uint32_t*)(b + o_rs),
                         (const uint16_t*)(b + o_it), (uint16_t*)dkv, acc, (float*)(b + o_hd), (float*)(b + o_tl),
                         (uint32_t)num_kv);
      hipLaunchKernelGGL(smla_bwd_dkv_fix_kernel, dim3((unsigned)((num_kv + 3) / 4)), dim3(256), 0, s,
                         (const uint32_t*)(b + o_rs), (const float*)(b + o_hd), (const float*)(b + o_tl),
                         (uint16_t*)dkv, acc, num_kv);
      err = hipGetLastError();
    }
  }
  if (err == hipSuccess && acc != nullptr && num_kv > 0) {
    hipLaunchKernelGGL(smla_bwd_dkv_out_kernel, dim3((unsigned)((num_kv + 3) / 4)), dim3(256), 0, s, acc,
                       (uint16_t*)dkv, num_kv);
    err = hipGetLastError();
  }
  if (err == hipSuccess && attn_sink) {
    hipLaunchKernelGGL(smla_bwd_dsink_kernel, dim3((unsigned)H), dim3(256), 0, s, (const float*)(b + o_dsp), (int)T,
                       (int)H, d_sink);
    err = hipGetLastError();
  }
  const hipError_t ferr = hipFreeAsync(ws, s);
  return (err == hipSuccess && ferr == hipSuccess) ? SMLA_OK : SMLA_ERR_LAUNCH;
}

}  // namespace

extern "C" int sparse_mla_backward(const void* q, const void* kv, const void* dout, const void* o, const float* lse,
                                   const int32_t* topk_indices, const float* attn_sink, float scale, void* dq,
                                   void* dkv, float* d_sink, int64_t T, int64_t H, int64_t num_kv, int64_t topk,
                                   void* stream) {
  return run_backward(q, kv, dout, o, lse, topk_indices, attn_sink, scale, dq, dkv, d_sink, T, H, num_kv, topk, 0,
                      stream);
}

extern "C" int sparse_mla_backward_chunked(const void* q, const void* kv, const void* dout, const void* o,
                                           const float* lse, const int32_t* topk_indices, const float* attn_sink,
                                           float scale, void* dq, void* dkv, float* d_sink, int64_t T, int64_t H,
                                           int64_t num_kv, int64_t topk, int64_t chunk_tokens, void* stream) {
  return run_backward(q, kv, dout, o, lse, topk_indices, attn_sink, scale, dq, dkv, d_sink, T, H, num_kv, topk,
                      chunk_tokens, stream);
}

extern "C" int sparse_mla_backward_i64(const void* q, const void* kv, const void* dout, const void* o,
                                       const float* lse, const int64_t* topk_indices, const float* attn_sink,
                                       float scale, void* dq, void* dkv, float* d_sink, int64_t T, int64_t H,
                                       int64_t num_kv, int64_t topk, int64_t chunk_tokens, void* stream) {
  int rc = bwd_check(q, kv, dout, o, lse, topk_indices, 8, attn_sink, scale, dq, dkv, d_sink, T, H, num_kv, topk,
                     chunk_tokens);
  if (rc != SMLA_OK) return rc;
  if (T == 0 || topk == 0)
    return run_backward(q, kv, dout, o, lse, nullptr, attn_sink, scale, dq, dkv, d_sink, T, H, num_kv, topk,
                        chunk_tokens, stream);
  int dev = 0;
  if (current_device(&dev) != SMLA_OK) return SMLA_ERR_NO_DEVICE;
  hipStream_t s = (hipStream_t)stream;
  // the rows as int32 row numbers (-1 where 0 <= v < num_kv fails in 64 bits), then the int32 backward
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
    rc = run_backward(q, kv, dout, o, lse, (const int32_t*)ws, attn_sink, scale, dq, dkv, d_sink, T, H, num_kv, topk,
                      chunk_tokens, stream);
  if (hipFreeAsync(ws, s) != hipSuccess && rc == SMLA_OK) rc = SMLA_ERR_LAUNCH;
  return rc;
}

extern "C" int sparse_mla_backward_fp8(const void* q, const void* kv, float kv_scale, const void* dout, const void* o,
                                       const float* lse, const int32_t* topk_indices, const float* attn_sink,
                                       float scale, void* dq, void* dkv, float* d_sink, int64_t T, int64_t H,
                                       int64_t num_kv, int64_t topk, int64_t chunk_tokens, void* stream) {
  int rc = bwd_check(q, kv, dout, o, lse, topk_indices, 4, attn_sink, scale, dq, dkv, d_sink, T, H, num_kv, topk,
                     chunk_tokens);
  if (rc != SMLA_OK) return rc;
  if (!isfinite(kv_scale) || !isfinite(scale * kv_scale)) return SMLA_ERR_BAD_SCALE;
  if (T == 0 || topk == 0 || num_kv == 0)  // no pool row is read
    return run_backward(q, kv, dout, o, lse, topk_indices, attn_sink, scale, dq, dkv, d_sink, T, H, num_kv, topk,
                        chunk_tokens, stream, kv_scale);
  int dev = 0;
  if (current_device(&dev) != SMLA_OK) return SMLA_ERR_NO_DEVICE;
  hipStream_t s = (hipStream_t)stream;
  // the pool as bf16 copies of its code values (exact), then the bf16 backward
  // with the dequant scale in the logits, dP and dq
  void* ws = nullptr;
  hipMemPool_t pool = scratch_pool(dev);
  if (pool == nullptr || hipMallocFromPoolAsync(&ws, (size_t)num_kv * kRowBytes, pool, s) != hipSuccess ||
      ws == nullptr) {
    (void)hipGetLastError();
    return SMLA_ERR_NO_MEMORY;
  }
  const int64_t n16 = num_kv * (kD / 16);
  const int64_t want = (n16 + 255) / 256;
  const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(smla_fp8_pool_decode_kernel, dim3(blocks), dim3(256), 0, s, (const uint8_t*)kv, (uint16_t*)ws,
                     n16);
  rc = hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
  if (rc == SMLA_OK)
    rc = run_backward(q, ws, dout, o, lse, topk_indices, attn_sink, scale, dq, dkv, d_sink, T, H, num_kv, topk,
                      chunk_tokens, stream, kv_scale);
  if (hipFreeAsync(ws, s) != hipSuccess && rc == SMLA_OK) rc = SMLA_ERR_LAUNCH;
  return rc;
}
