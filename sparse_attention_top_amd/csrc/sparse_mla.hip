// Sparse MLA prefill forward (DeepSeek-V4) for MI355X / gfx950 (CDNA4).
//
// Operation: "[Triton/Gluon] [GFX950][DSV4] Sparse MLA training backward"
// (aiter PR #4766), section "Contract" -- per token t and head h, softmax of
// scale * q.k over the valid gathered rows of a shared bf16 pool (K == V),
// with an optional per-head sink logit in the denominator only; outputs bf16
// o and a sink-inclusive natural-log lse. The C ABI is in
// include/sparse_mla.h.
//
// Kernel structure (one workgroup per token and group of heads):
//   1. the token's top-k row is read and its valid slots (0 <= idx < num_kv,
//      one unsigned compare) are compacted into an LDS list -- invalid slots
//      are never dereferenced, so NaN/Inf in unused pool rows cannot reach
//      the output (the fix described on "[Triton/Gluon] [CI] [gfx942] Tuned
//      sparse MLA prefill for DSv4.1-Flash TP4; fix attn_sink in Triton
//      fallback" (aiter PR #6002), description);
//   2. tiles of 32 valid rows are gathered global->LDS with the CDNA4
//      LDS-DMA load (one wave instruction moves one whole 1 KiB row), into a
//      ring of NBUF buffers, so that one gather serves every head of the token
//      and both contractions;
//   3. S^T = K Q^T on bf16 MFMA (16x16x32, fp32 accumulate), K read from LDS;
//   4. online softmax in base 2 (scale * log2 e folded into one multiply),
//      with lazy rescaling: the reference max only moves when a tile's max
//      exceeds it by more than 2^8, which is exact because the final
//      normalisation uses the same reference;
//   5. O^T += V^T P^T on bf16 MFMA, V read from the same LDS tile with the
//      gfx950 transposing LDS load, P rounded to bf16;
//   6. the sink is folded into the max and the denominator at the end, o is
//      rounded to bf16 and lse converted back to natural log.
//
// Invalid (tail) rows of a partial tile are zero-filled in LDS and their
// logits forced to -inf, so stale LDS contents never reach the output.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sparse_mla.h"

namespace {

constexpr int kD = SPARSE_MLA_HEAD_DIM;  // 512
constexpr int kRowBytes = kD * 2;        // one bf16 row = 1 KiB
constexpr int kRowStride = kRowBytes + 16;  // LDS row pitch: 16 B of padding spreads rows over the banks
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
#define LDS_AS __attribute__((address_space(3)))

struct Params {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* topk;
  const float* sink;
  uint16_t* out;
  float* lse;
  int T;
  int H;
  uint32_t nkv;  // min(num_kv, 2^31): slot valid iff (uint32)idx < nkv
  int topk_n;
  int head_groups;
  float scale_log2;  // scale * log2(e)
};

template <int NW, int NBUF>
struct Smem {
  uint8_t tile[NBUF][kBK][kRowStride];
  int32_t list[kListCap];
  int32_t wcount[NW];
};

// Optimisation barrier on a per-tile base address: keeps loop strength
// reduction from hoisting one address register per unrolled offset (the
// constant offsets then fold into the LDS instructions' offset fields).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(LDS_AS const void*)p; }

template <typename T>
__device__ __forceinline__ T lds_load(uint32_t addr) {
  return *(LDS_AS const T*)(uintptr_t)addr;
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most n of this wave's vector-memory operations are
// outstanding (n rounded down to an encodable step; waiting more is safe).
__device__ __forceinline__ void wait_vmcnt_le(int n) {
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

// Compact the valid entries of trow[0, len) into sm.list (order kept).
// Returns the count (uniform across the workgroup).
template <int NW, int NBUF>
__device__ int compact_segment(const int32_t* __restrict__ trow, int len, uint32_t nkv, Smem<NW, NBUF>& sm,
                               int lane, int w) {
  int base = 0;
  for (int c0 = 0; c0 < len; c0 += NW * 64) {
    const int pos = c0 + w * 64 + lane;
    const int raw = pos < len ? trow[pos] : -1;
    const bool valid = (uint32_t)raw < nkv;
    const uint64_t bal = __ballot(valid);
    const int rank = lane_rank(bal);
    const int wc = __popcll(bal);
    if constexpr (NW == 1) {
      if (valid) sm.list[base + rank] = raw;
      base += wc;
    } else {
      if (lane == 0) sm.wcount[w] = wc;
      lds_barrier();
      int off = 0, tot = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const int ci = __builtin_amdgcn_readfirstlane(sm.wcount[i]);
        off += (i < w) ? ci : 0;
        tot += ci;
      }
      if (valid) sm.list[base + off + rank] = raw;
      base += tot;
      lds_barrier();
    }
  }
  return __builtin_amdgcn_readfirstlane(base);
}

template <int NW>
__device__ __forceinline__ int tile_rows(int i, int n) { return min(kBK, n - i * kBK); }

// Number of LDS-DMA loads this wave issues for tile i.
template <int NW>
__device__ __forceinline__ int tile_dma(int i, int n, int w) {
  constexpr int RPW = kBK / NW;
  return min(RPW, max(0, tile_rows<NW>(i, n) - w * RPW));
}

// Issue the gather of tile i (rows list[32 i, 32 i + cnt)) into its ring
// buffer; rows past cnt are zero-filled. Each wave moves rows
// [w RPW, (w+1) RPW): one LDS-DMA instruction per row, lane L moving bytes
// [16 L, 16 L + 16) of the row.
template <int NW, int NBUF>
__device__ __forceinline__ void issue_tile(int i, int n, Smem<NW, NBUF>& sm, const uint16_t* __restrict__ kv,
                                           int lane, int w) {
  constexpr int RPW = kBK / NW;
  const int buf = i % NBUF;
  const int cnt = tile_rows<NW>(i, n);
  const int r0 = w * RPW;
  const int my = (lane < RPW && r0 + lane < cnt) ? sm.list[i * kBK + r0 + lane] : 0;
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = r0 + rr;
    uint8_t* dst = &sm.tile[buf][r][0];
    if (r < cnt) {
      const int row = __builtin_amdgcn_readlane(my, rr);
      const uint16_t* src = kv + (size_t)(uint32_t)row * kD + 8 * lane;
      __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)dst, 16, 0, 0);
    } else {
      *(u32x4*)(dst + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int NHT, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void smla_fwd_kernel(const Params p) {
  __shared__ __attribute__((aligned(16))) Smem<NW, NBUF> sm;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // 16-lane group
  const int li = lane & 15;  // index within the group

  const int v = xcd_remap(blockIdx.x, gridDim.x);
  const int t = p.T - 1 - v / p.head_groups;  // latest (heaviest) tokens first
  const int hg = v % p.head_groups;
  const int head_base = (hg * NW + w) * (NHT * 16);

  // Q^T fragments (MFMA B operand): lane holds q[t, head, 32k + 8g .. +8).
  bf16x8 qf[NHT][16];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int head = head_base + ht * 16 + li;
    if (head < p.H) {
      const bf16x8* src = (const bf16x8*)(p.q + ((size_t)t * p.H + head) * kD + 8 * g);
#pragma unroll
      for (int k = 0; k < 16; ++k) qf[ht][k] = src[4 * k];
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) qf[ht][k] = bf16x8{};
    }
  }

  f32x4 acc[NHT][32];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) acc[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[NHT], l_part[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    m_ref[ht] = -INFINITY;
    l_part[ht] = 0.f;
  }

  const int32_t* trow = p.topk + (size_t)t * p.topk_n;
  int n_total = 0;
  for (int seg0 = 0; seg0 < p.topk_n; seg0 += kListCap) {
    if (seg0 > 0 && NW > 1) lds_barrier();  // previous segment's list fully consumed
    const int n = compact_segment<NW, NBUF>(trow + seg0, min(kListCap, p.topk_n - seg0), p.nkv, sm, lane, w);
    n_total += n;
    const int ntiles = (n + kBK - 1) / kBK;

#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
      if (i < ntiles) issue_tile<NW, NBUF>(i, n, sm, p.kv, lane, w);

    for (int j = 0; j < ntiles; ++j) {
      int after = 0;
#pragma unroll
      for (int i = 1; i <= NBUF - 2; ++i)
        if (j + i < ntiles) after += tile_dma<NW>(j + i, n, w);
      wait_vmcnt_le(after);
      if constexpr (NW > 1) lds_barrier();
      if (j + NBUF - 1 < ntiles) issue_tile<NW, NBUF>(j + NBUF - 1, n, sm, p.kv, lane, w);

      const uint32_t tb = lds_addr(&sm.tile[j % NBUF][0][0]);
      const int cnt = tile_rows<NW>(j, n);

      // ---- S^T = K Q^T (two 16-slot halves) ----
      // K fragment (MFMA A operand): lane holds K[slot sh*16 + li][32k + 8g .. +8),
      // software-pipelined KPF k-steps ahead; the scheduler fence keeps the
      // loads from being hoisted further (register pressure).
      f32x4 s[2][NHT];
#pragma unroll
      for (int sh = 0; sh < 2; ++sh)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) s[sh][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      constexpr int KPF = 2;
      bf16x8 kf[KPF + 1][2];
      const uint32_t krow = opaque(tb + li * kRowStride + 16 * g);
#pragma unroll
      for (int k = 0; k < 16 + KPF; ++k) {
        if (k < 16) {
          kf[k % (KPF + 1)][0] = lds_load<bf16x8>(krow + 64 * k);
          kf[k % (KPF + 1)][1] = lds_load<bf16x8>(krow + 16 * kRowStride + 64 * k);
        }
        if (k >= KPF) {
          const int kk = k - KPF;
#pragma unroll
          for (int sh = 0; sh < 2; ++sh)
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht)
              s[sh][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk % (KPF + 1)][sh], qf[ht][kk], s[sh][ht], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- online softmax (base 2) ----
      float x[NHT][2][4], tmax[NHT];
      bool need = false;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        float mx = -INFINITY;
#pragma unroll
        for (int sh = 0; sh < 2; ++sh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int slot = sh * 16 + 4 * g + i;
            const float xv = slot < cnt ? s[sh][ht][i] * p.scale_log2 : -INFINITY;
            x[ht][sh][i] = xv;
            mx = fmaxf(mx, xv);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        tmax[ht] = mx;
        need |= mx > m_ref[ht] + kLazyTau;
      }
      if (__ballot(need) != 0ull) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          const float m_new = fmaxf(m_ref[ht], tmax[ht]);
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref[ht] - m_new);
          m_ref[ht] = m_new;
          l_part[ht] *= alpha;
          // in place, one accumulator register at a time (the accumulators
          // live in AGPRs; a plain vector multiply would stage all of them
          // through VGPRs)
#pragma unroll
          for (int dt = 0; dt < 32; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float e = acc[ht][dt][i];
              float tmp;
              asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                           : "+a"(e), "=&v"(tmp)
                           : "v"(alpha));
              acc[ht][dt][i] = e;
            }
        }
      }
      bf16x8 pk[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const float mu = (m_ref[ht] == -INFINITY) ? 0.f : m_ref[ht];
        float ls = 0.f;
#pragma unroll
        for (int sh = 0; sh < 2; ++sh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = __builtin_amdgcn_exp2f(x[ht][sh][i] - mu);
            ls += pv;
            pk[ht][sh * 4 + i] = (__bf16)pv;
          }
        l_part[ht] += ls;
      }

      // ---- O^T += V^T P^T ----
      // V^T fragment (MFMA A operand): lane holds V[rows 4g..4g+3 and
      // 16+4g..16+4g+3][16 dt + li], via two transposing LDS reads.
      // this lane addresses row 4g + li/4 (and that + 16), bytes 8 (li & 3) + 32 dt
      const uint32_t vrow = opaque(tb + (4 * g + (li >> 2)) * kRowStride + 8 * (li & 3));
      constexpr int VPF = 3;
      bf16x4 vf[VPF + 1][2];
#pragma unroll
      for (int dt = 0; dt < 32 + VPF; ++dt) {
        if (dt < 32) {
          vf[dt % (VPF + 1)][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(uintptr_t)(vrow + 32 * dt));
          vf[dt % (VPF + 1)][1] =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(uintptr_t)(vrow + 16 * kRowStride + 32 * dt));
        }
        if (dt >= VPF) {
          const int d = dt - VPF;
          const bf16x4 v0 = vf[d % (VPF + 1)][0], v1 = vf[d % (VPF + 1)][1];
          const bf16x8 a = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) acc[ht][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pk[ht], acc[ht][d], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  (void)n_total;

  // ---- finalise: fold the sink, normalise, store ----
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    float lsum = l_part[ht];
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const int head = head_base + ht * 16 + li;
    const bool hv = head < p.H;
    const float sk = (p.sink != nullptr && hv) ? p.sink[head] : -INFINITY;
    const bool has_sink = !(sk == -INFINITY);
    float oscale, lse_v;
    if (lsum == 0.f) {  // no valid slot carried any mass
      oscale = 0.f;
      lse_v = sk;
    } else {
      const float mu = m_ref[ht];
      const float s2 = sk * kLog2e;
      const float mf = has_sink ? fmaxf(mu, s2) : mu;
      const float a = __builtin_amdgcn_exp2f(mu - mf);
      const float lf = lsum * a + (has_sink ? __builtin_amdgcn_exp2f(s2 - mf) : 0.f);
      oscale = a / lf;
      lse_v = (mf + __builtin_amdgcn_logf(lf)) * kLn2;
    }
    if (hv) {
      uint16_t* orow = p.out + ((size_t)t * p.H + head) * kD + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const f32x4 o = acc[ht][dt] * oscale;
        *(bf16x4*)(orow + 16 * dt) = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
      }
      if (g == 0) p.lse[(size_t)t * p.H + head] = lse_v;
    }
  }
}

struct Variant {
  int nht, nw;
  const char* name;
};

// Small head counts (H <= 16): one wave per token, one 16-head tile; the
// gather dominates. More heads: 32 heads per wave (each K/V fragment read from
// LDS feeds two MFMAs), up to four waves (128 heads) per workgroup.
Variant pick_variant(int64_t H) {
  if (H <= 16) return {1, 1, "smla_fwd_kernel<1, 1, 2>"};
  const int64_t waves = (H + 31) / 32;
  if (waves <= 1) return {2, 1, "smla_fwd_kernel<2, 1, 2>"};
  if (waves <= 2) return {2, 2, "smla_fwd_kernel<2, 2, 3>"};
  return {2, 4, "smla_fwd_kernel<2, 4, 3>"};
}

template <int NHT, int NW, int NBUF>
hipError_t launch(const Params& p, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((smla_fwd_kernel<NHT, NW, NBUF>), dim3(blocks), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

}  // namespace

extern "C" int sparse_mla_prefill(const void* q, const void* kv, const int32_t* topk_indices, const float* attn_sink,
                                  float scale, void* out, float* lse, int64_t T, int64_t H, int64_t num_kv,
                                  int64_t topk, void* stream) {
  if (T < 0 || H < 1 || num_kv < 0 || topk < 0) return SMLA_ERR_BAD_SIZE;
  if (T > INT32_MAX || H > INT32_MAX || topk > INT32_MAX) return SMLA_ERR_BAD_SIZE;
  if (!isfinite(scale)) return SMLA_ERR_BAD_SCALE;
  if (T == 0) return SMLA_OK;
  const Variant var = pick_variant(H);
  const int64_t heads_per_wg = (int64_t)var.nht * 16 * var.nw;
  const int64_t head_groups = (H + heads_per_wg - 1) / heads_per_wg;
  if (T * head_groups > INT32_MAX) return SMLA_ERR_BAD_SIZE;
  if (T > INT64_MAX / H / kD || T > INT64_MAX / (topk > 0 ? topk : 1)) return SMLA_ERR_BAD_SIZE;
  if (!q || !out || !lse) return SMLA_ERR_NULL_POINTER;
  if (topk > 0 && !topk_indices) return SMLA_ERR_NULL_POINTER;
  if (topk > 0 && num_kv > 0 && !kv) return SMLA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(out, 16) || (kv && !aligned(kv, 16))) return SMLA_ERR_MISALIGNED;
  if (!aligned(lse, 4) || (topk_indices && !aligned(topk_indices, 4)) || (attn_sink && !aligned(attn_sink, 4)))
    return SMLA_ERR_MISALIGNED;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return SMLA_ERR_NO_DEVICE;
  }

  Params p;
  p.q = (const uint16_t*)q;
  p.kv = (const uint16_t*)kv;
  p.topk = topk_indices;
  p.sink = attn_sink;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.T = (int)T;
  p.H = (int)H;
  p.nkv = (uint32_t)(num_kv < ((int64_t)1 << 31) ? num_kv : ((int64_t)1 << 31));
  if (topk == 0 || !kv) p.nkv = 0;
  p.topk_n = (int)topk;
  p.head_groups = (int)head_groups;
  p.scale_log2 = scale * kLog2e;
  const int blocks = (int)(T * head_groups);
  hipStream_t s = (hipStream_t)stream;
  hipError_t err;
  if (var.nht == 1) err = launch<1, 1, 2>(p, blocks, s);
  else if (var.nw == 1) err = launch<2, 1, 2>(p, blocks, s);
  else if (var.nw == 2) err = launch<2, 2, 3>(p, blocks, s);
  else err = launch<2, 4, 3>(p, blocks, s);
  return err == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

extern "C" const char* sparse_mla_status_string(int status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case SMLA_ERR_BAD_SIZE: return "invalid size (T<0, H<1, num_kv<0, topk<0, or overflow)";
    case SMLA_ERR_MISALIGNED: return "misaligned pointer (q, kv, out need 16 bytes; lse, topk, sink need 4)";
    case SMLA_ERR_BAD_SCALE: return "scale must be finite";
    case SMLA_ERR_NO_DEVICE: return "no usable HIP device";
    case SMLA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" const char* sparse_mla_kernel_name(int64_t H) {
  if (H < 1) return nullptr;
  return pick_variant(H).name;
}

extern "C" int sparse_mla_version(void) { return 100; }
