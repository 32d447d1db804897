// Paged decode attention for gfx950.
//
// "KV-Cache Optimization Techniques", section "PagedAttention", eq. 1: the new
// query token of a sequence attends over the K/V rows of its pages, gathered
// in logical order through the sequence's page table:
//   out_j = softmax(scale * q_j K^T) V,  query head j reading KV head j / g
// (section "Multi-Query and Grouped-Query Caching", eq. 7).  Quantized pools
// hold codes with a per-token scale and zero point (section "KV-Cache
// Quantization", eq. 3; INT8 and INT4 codes, or FP8 e4m3 values with zero
// point 0), dequantized here: q.k = s*(q.c) + z*sum(q) and
// sum_t p_t v_t = sum_t (p_t s_t) c_t + sum_t p_t z_t.
//
// Work decomposition.  A workgroup owns one (sequence, KV head) pair and one
// range of logical blocks (a split); its W wavefronts each stream a
// contiguous share of those pages with a register ring of DEPTH pages in
// flight, keep an online softmax in float32 (running max m, running sum l,
// rescaled accumulator), and merge in LDS at the end.  With several splits
// the merged partials (o, m, l) go to a workspace and merge_kernel combines
// them by log-sum-exp.  Scores live in log2 units (scale * log2 e folded in)
// so every exponential is one v_exp_f32.
//
// Matrix-core path (g >= 4): per 16-token sub-tile, S^T = K q^T on
// v_mfma_f32_16x16x32 (K rows are the A operand, loaded straight from HBM
// with 16-byte loads: each lane holds 8 channels of one token), then
// O^T += V^T P^T on v_mfma_f32_16x16x16 (P = 16) or 16x16x32 (P = 32).  The
// S^T accumulator layout (lane: head l%16, tokens 4*(l/16)..+3) is exactly the
// B-operand layout P^T needs, and the O^T accumulator keeps head l%16 in the
// same lane, so the whole online softmax is lane-local except the max over
// tokens (two cross-lane steps).  V is stored transposed per (page, head) so
// each lane's V^T operand is one contiguous load.  Query heads are padded to
// 16 per tile; NT tiles cover g up to 16*NT.
//
// Vector-ALU path (g < 4): four lanes per token row split the channels for
// the dot products; probabilities are broadcast through LDS for P.V.
#pragma once
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "kvp.h"

namespace kvp {

struct DecodeArgs {
  const uint16_t* q;
  const void* k_pool;
  const void* v_pool;
  const uint16_t* k_meta;
  const uint16_t* v_meta;
  const int32_t* bt;
  const int32_t* ctx_lens;
  uint16_t* out;
  float* part_o;
  float* part_ml;
  int32_t num_seqs, max_blocks, num_kv_heads, num_q_heads, group, num_pages, num_splits,
      pages_per_split;
  int32_t ctx_cap;
  int32_t sink_tokens, window_tokens;  // window_tokens > 0: attend only to the kept set
  int32_t write_partials;  // 1: store (o, m, l) per split; 0: store the bf16 output
  float scale_log2;  // scale * log2(e)
  const int32_t* sched;    // balanced schedule (bin starts at word 8), or null
  int32_t items_off;       // word offset of its item records
  int32_t num_items, num_slots, num_bins;
};

// The tokens a sequence of n attends to.  Without a window, 0..n-1.  With a
// window ("KV-Cache Optimization Techniques", section "Token Eviction
// Strategies", eq. 5, attention sinks plus a recent window; section "Sliding
// Window Cache", eq. 6, when there are no sinks) and sink + window < n, only
// t < sink or t >= n - window.  The pages streamed are the virtual block list
// "sink blocks, then window blocks": virtual block v is logical block v below
// sink_blk and win_first + (v - sink_blk) from there on; blocks in between hold
// only dropped tokens and are never read (their table entries may be -1).
struct WorkRange {
  int b, h, s, ctx;
  int slot;                // scheduled item: partial slot, -1 for the direct output
  int kb0, cnt;            // this wave's virtual blocks [kb0, kb0 + cnt)
  int sink_blk, win_first;
  int sink_end, win_start;  // kept: t < ctx and (t < sink_end or t >= win_start)
  __device__ __forceinline__ int logical(int v) const {
    return v < sink_blk ? v : win_first + (v - sink_blk);
  }
};

// Rows of one page that take part (relative token bounds of the kept set).
struct PageMask {
  int end, sink_end, win_start;
  bool partial;  // some row of the page is not kept
  __device__ __forceinline__ bool valid(int r) const {
    return r < end && (r < sink_end || r >= win_start);
  }
};

template <int P>
__device__ __forceinline__ PageMask page_mask(const WorkRange& w, int lblk) {
  const int base = lblk * P;
  PageMask m;
  m.end = w.ctx - base;
  m.sink_end = w.sink_end - base;
  m.win_start = w.win_start - base;
  m.partial = !(m.end >= P && (m.sink_end >= P || m.win_start <= 0));
  return m;
}

// Which (sequence, KV head, split) this workgroup owns and which contiguous
// run of virtual blocks [kb0, kb0 + cnt) wave `wave` streams.
//
// Workgroups are handed to the eight XCDs round robin (workgroup i to XCD
// i mod 8), so the index order decides each XCD's share of the work.  The KV
// head varies fastest (the heads of one sequence carry equal work), then the
// sequence, and the split slowest: every XCD gets the same mix of long and
// short sequences and of first and last splits, and the always-full first
// splits are dispatched first.  (With the split fastest and eight KV heads,
// an even split count gave each XCD a single split index: half the XCDs
// streamed every sequence's first pages while the other half idled.)
// Sequence b's streamed block list (see WorkRange) and its length.
template <int P>
__device__ __forceinline__ int sequence_blocks(const DecodeArgs& a, WorkRange& w) {
  int ctx = a.ctx_lens[w.b];
  ctx = min(max(ctx, 0), a.ctx_cap);
  w.ctx = ctx;
  const int nblk = (ctx + P - 1) / P;
  int nvirt = nblk;
  w.sink_blk = nblk;
  w.win_first = nblk;
  w.sink_end = ctx;
  w.win_start = ctx;
  if (a.window_tokens > 0 && int64_t(a.sink_tokens) + a.window_tokens < int64_t(ctx)) {
    w.sink_end = a.sink_tokens;
    w.win_start = ctx - a.window_tokens;
    w.sink_blk = (a.sink_tokens + P - 1) / P;
    w.win_first = max(w.win_start / P, w.sink_blk);
    nvirt = w.sink_blk + (nblk - w.win_first);
  }
  return nvirt;
}

// Wave `wave` of W takes a contiguous share of virtual blocks [blk0, blk1).
__device__ __forceinline__ void wave_share(WorkRange& w, int blk0, int blk1, int wave, int W) {
  const int n = max(blk1 - blk0, 0);
  const int cw = (n + W - 1) / W;
  w.kb0 = blk0 + wave * cw;
  w.cnt = max(0, min(cw, blk1 - w.kb0));
}

// Which (sequence, KV head, split) this workgroup owns and which contiguous
// run of virtual blocks [kb0, kb0 + cnt) wave `wave` streams.
//
// Workgroups are handed to the eight XCDs round robin (workgroup i to XCD
// i mod 8), so the index order decides each XCD's share of the work.  The KV
// head varies fastest (the heads of one sequence carry equal work), then the
// sequence, and the split slowest: every XCD gets the same mix of long and
// short sequences and of first and last splits, and the always-full first
// splits are dispatched first.  (With the split fastest and eight KV heads,
// an even split count gave each XCD a single split index: half the XCDs
// streamed every sequence's first pages while the other half idled.)
template <int P>
__device__ __forceinline__ WorkRange work_range(const DecodeArgs& a, int wave, int W) {
  WorkRange w;
  int item = blockIdx.x;
  w.h = item % a.num_kv_heads;
  item /= a.num_kv_heads;
  w.b = item % a.num_seqs;
  w.s = item / a.num_seqs;
  w.slot = -1;
  const int nvirt = sequence_blocks<P>(a, w);
  const int blk0 = w.s * a.pages_per_split;
  wave_share(w, blk0, min(blk0 + a.pages_per_split, nvirt), wave, W);
  return w;
}

// A schedule item names a sequence and KV head of this call and a partial
// slot within the workspace (or -1); anything else is skipped.
__device__ __forceinline__ bool item_valid(const DecodeArgs& a, int i) {
  const int32_t* it = a.sched + a.items_off + int64_t(i) * 8;
  return unsigned(it[0]) < unsigned(a.num_seqs) && unsigned(it[1]) < unsigned(a.num_kv_heads) &&
         it[4] >= -1 && it[4] < a.num_slots;
}

// Item `i` of a balanced schedule: sequence, KV head, streamed blocks
// [first, end) (clipped to the device length), partial slot.
template <int P>
__device__ __forceinline__ WorkRange item_range(const DecodeArgs& a, int i, int wave, int W) {
  const int32_t* it = a.sched + a.items_off + int64_t(i) * 8;
  WorkRange w;
  w.b = it[0];
  w.h = it[1];
  w.s = 0;
  w.slot = it[4];
  const int nvirt = sequence_blocks<P>(a, w);
  wave_share(w, max(it[2], 0), min(it[3], nvirt), wave, W);
  return w;
}

// Merge the W wavefronts' (m, l, o) partials held in LDS and store either the
// final bfloat16 output (one split) or this split's normalized partial.
template <int D, bool SCHED>
__device__ __forceinline__ void combine_and_store(const DecodeArgs& a, const WorkRange& wr,
                                                  const float* sm_o, const float* sm_m,
                                                  const float* sm_l, int W, int HP) {
  const int g = a.group;
  for (int e = threadIdx.x; e < g * D; e += blockDim.x) {
    const int j = e / D, d = e - j * D;
    float M = -INFINITY;
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w * HP + j]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
      for (int w = 0; w < W; ++w) {
        const float mw = sm_m[w * HP + j];
        if (mw != -INFINITY) {
          const float f = fast_exp2(mw - M);
          L += sm_l[w * HP + j] * f;
          O += sm_o[(w * g + j) * D + d] * f;
        }
      }
    }
    const float res = L > 0.0f ? O / L : 0.0f;
    const int64_t row = int64_t(wr.b) * a.num_q_heads + int64_t(wr.h) * g + j;
    const bool direct = SCHED ? wr.slot < 0 : !a.write_partials;
    if (direct) {
      a.out[row * D + d] = f32_to_bf16_rne(res);
    } else {
      const int64_t pr = SCHED ? int64_t(wr.slot) * g + j : row * a.num_splits + wr.s;
      a.part_o[pr * D + d] = res;
      if (d == 0) {
        a.part_ml[pr * 2] = M;
        a.part_ml[pr * 2 + 1] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core kernel.
template <int F, int P, int D>
struct MfmaShape {
  using FI = FmtInfo<F>;
  static constexpr int T = P / 16;          // 16-token sub-tiles per page
  static constexpr int KK = D / 32;         // 16x16x32 steps over the head dim
  static constexpr int NC = D / 16;         // 16-channel output chunks
  static constexpr int EV = 4 * T;          // tokens per lane in P.V
  static constexpr int RB = D * FI::bits / 8;  // bytes of one stored token row
  // K bytes a lane holds per 16-token sub-tile.  The four lane groups (gq)
  // read interleaved 16-byte pieces, so each load instruction covers whole
  // 64-byte spans of a token row: bfloat16, KK pieces of 8 channels 32
  // apart; 8-bit codes, D/64 pieces of 16 channels 64 apart; INT4, D/4
  // contiguous channels (one piece of D/8 bytes).
  static constexpr int KB = FI::quant ? (D / 4) * FI::bits / 8 : 16 * KK;
  // q channel of k-step kk in lane group gq, matching the K pieces above
  __device__ static constexpr int q_channel(int kk, int gq) {
    return F == kBF16 ? 32 * kk + 8 * gq
         : F == kI4   ? (D / 4) * gq + 8 * kk
                      : 64 * (kk >> 1) + 16 * gq + 8 * (kk & 1);
  }
  __device__ static constexpr int k_lane_offset(int gq) { return F == kI4 ? gq * KB : 16 * gq; }
  static constexpr int KLB = KB >= 16 ? 16 : KB;  // bytes per K load
  static constexpr int KN = KB / KLB;             // K loads per sub-tile
  // V^T bytes a lane holds per 16-channel chunk: EV tokens of one channel (for
  // INT4 the byte of the channel pair holding it)
  static constexpr int VB = F == kBF16 ? EV * 2 : EV;
};

template <int BYTES> struct LoadT;
template <> struct LoadT<4> { using type = uint32_t; };
template <> struct LoadT<8> { using type = uint2; };
template <> struct LoadT<16> { using type = uint4; };

template <int F, int P, int D>
struct PageRegs {
  using S = MfmaShape<F, P, D>;
  typename LoadT<S::KLB>::type k[S::T][S::KN];
  typename LoadT<S::VB>::type v[S::NC];
  uint4 km[FmtInfo<F>::quant ? S::T : 1];
  uint4 vm[FmtInfo<F>::quant ? S::T : 1];
  int phys;  // page id, -1 when the table entry is out of range
};

// Largest workgroup each instance is compiled for: four wavefronts, one per
// SIMD, which is what kvp_decode_plan asks for (fewer when the LDS merge
// buffer of a large group would not fit).
constexpr int mfma_max_threads(int, int, int) { return 256; }
constexpr int valu_max_threads(int, int, int) { return 256; }

// Operand types of the matrix-core path: q^T and K as float16 (quantized
// pools: exact code values) or bfloat16; P.V operands are four-wide for
// 16-token pages.
template <int F, int P, int D>
struct MfmaOps {
  static constexpr bool Q = FmtInfo<F>::quant;
  using A = typename std::conditional<Q, f16x8_t, bf16x8_t>::type;
  using PV = typename std::conditional<
      MfmaShape<F, P, D>::T == 1, typename std::conditional<Q, f16x4_t, bf16x4_t>::type,
      A>::type;
};

// Per-lane byte offsets inside a (page, head) tile: K rows of each 16-token
// sub-tile, the V^T row, the metadata of the lane's tokens.
template <int F, int P, int D>
struct MfmaLaneOffsets {
  int koff[MfmaShape<F, P, D>::T];
  int voff, moff;
};
template <int F, int P, int D>
__device__ __forceinline__ MfmaLaneOffsets<F, P, D> mfma_lane_offsets(int r, int gq) {
  using S = MfmaShape<F, P, D>;
  MfmaLaneOffsets<F, P, D> o;
#pragma unroll
  for (int st = 0; st < S::T; ++st) {
    // sub-tile st, MFMA row r -> token; with two sub-tiles the rows are
    // interleaved so a lane's eight P.V tokens are contiguous.
    const int tok = (S::T == 1) ? r : 8 * (r >> 2) + 4 * st + (r & 3);
    o.koff[st] = tok * S::RB + S::k_lane_offset(gq);
  }
  // V^T tile: [D][P] elements, or [D/2][P] bytes for INT4 (channel pairs)
  o.voff = F == kBF16 ? (r * P + S::EV * gq) * 2 : (F == kI4 ? (r >> 1) * P : r * P) + S::EV * gq;
  o.moff = S::EV * gq * 4;
  return o;
}

// q^T of an item as the B operand of S^T = K q^T: lane (r, gq) holds head
// nt*16 + r (zero past the group), the 8 channels q_channel(kk, gq) of each
// k-step; for quantized pools float16 values and, for the zero-point term,
// qsum = the sum of the head's channels (float32, from the bfloat16 values;
// for INT4 from their float16 operand values).
// A negative scale is applied as |scale| on -q (exact), so that scores are
// always |scale| times a raw dot product and their maximum is the raw one's.
// In two steps: the loads (raw bfloat16 words), then the conversion.
template <int F, int P, int D, int NT>
__device__ __forceinline__ void mfma_q_raw(const DecodeArgs& a, int b, int h, int r, int gq,
                                           uint4 (&raw)[NT][MfmaShape<F, P, D>::KK]) {
  using S = MfmaShape<F, P, D>;
  const int g = a.group;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int jj = nt * 16 + r;
    const bool live = jj < g;
    const uint16_t* qrow = a.q + (int64_t(b) * a.num_q_heads + int64_t(h) * g + (live ? jj : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < S::KK; ++kk)
      raw[nt][kk] = live ? *reinterpret_cast<const uint4*>(qrow + S::q_channel(kk, gq))
                         : make_uint4(0, 0, 0, 0);
  }
}
template <int F, int P, int D, int NT>
__device__ __forceinline__ void mfma_q_convert(const DecodeArgs& a,
                                               const uint4 (&raw)[NT][MfmaShape<F, P, D>::KK],
                                               typename MfmaOps<F, P, D>::A (&qop)[NT][MfmaShape<F, P, D>::KK],
                                               float (&qsum)[NT]) {
  using S = MfmaShape<F, P, D>;
  constexpr bool Q = FmtInfo<F>::quant, ZP = FmtInfo<F>::zero;
  const uint32_t qflip = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float qs = 0.0f;
#pragma unroll
    for (int kk = 0; kk < S::KK; ++kk) {
      uint4 w = raw[nt][kk];
      w.x ^= qflip;
      w.y ^= qflip;
      w.z ^= qflip;
      w.w ^= qflip;
      if constexpr (!Q) {
        qop[nt][kk] = __builtin_bit_cast(bf16x8_t, w);
      } else {
        const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
        f16x8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = F == kI4 ? kI4KSlot(e) : e;  // the K operand's channel order
          const float f = bf16_to_f32((w4[c >> 1] >> (16 * (c & 1))) & 0xffffu);
          v[e] = (_Float16)f;
          // INT4: the sum of the operand's own values, which the K codes'
          // offset is removed with (the same as f's unless q is tiny)
          qs += F == kI4 ? float(v[e]) : f;
        }
        qop[nt][kk] = v;
      }
    }
    qsum[nt] = ZP ? group4_sum(qs) : 0.0f;
  }
}
template <int F, int P, int D, int NT>
__device__ __forceinline__ void mfma_load_q(const DecodeArgs& a, int b, int h, int r, int gq,
                                            typename MfmaOps<F, P, D>::A (&qop)[NT][MfmaShape<F, P, D>::KK],
                                            float (&qsum)[NT]) {
  uint4 raw[NT][MfmaShape<F, P, D>::KK];
  mfma_q_raw<F, P, D, NT>(a, b, h, r, gq, raw);
  mfma_q_convert<F, P, D, NT>(a, raw, qop, qsum);
}

// Issue the loads of one (page, head) tile into a ring slot.  phys is the raw
// table entry: out of range -> the slot is marked absent (phys = -1) and
// page 0 is read in its place, so the load pattern stays fixed.
template <int F, int P, int D>
__device__ __forceinline__ void mfma_load_page(const DecodeArgs& a, int phys, int h,
                                               const MfmaLaneOffsets<F, P, D>& o,
                                               PageRegs<F, P, D>& R) {
  using S = MfmaShape<F, P, D>;
  using KLoad = typename LoadT<S::KLB>::type;
  using VLoad = typename LoadT<S::VB>::type;
  constexpr int vstride = F == kBF16 ? 16 * P * 2 : (F == kI4 ? 8 * P : 16 * P);
  const bool ok = unsigned(phys) < unsigned(a.num_pages);
  R.phys = ok ? phys : -1;
  const int64_t tile = int64_t(ok ? phys : 0) * a.num_kv_heads + h;
  const size_t tile_bytes = size_t(P) * S::RB;
  const char* kp = static_cast<const char*>(a.k_pool) + tile * tile_bytes;
  const char* vp = static_cast<const char*>(a.v_pool) + tile * tile_bytes;
  // the per-token metadata first: the V scales decide the page's operand
  // offset before its scores are computed, and waiting for them then does
  // not wait for the page's codes
  if constexpr (FmtInfo<F>::quant) {
    const char* km = reinterpret_cast<const char*>(a.k_meta) + tile * (P * 4);
    const char* vm = reinterpret_cast<const char*>(a.v_meta) + tile * (P * 4);
#pragma unroll
    for (int st = 0; st < S::T; ++st) {
      R.vm[st] = load_stream<uint4>(vm + o.moff + st * 16);
      R.km[st] = load_stream<uint4>(km + o.moff + st * 16);
    }
  }
#pragma unroll
  for (int st = 0; st < S::T; ++st)
#pragma unroll
    for (int i = 0; i < S::KN; ++i) R.k[st][i] = load_stream<KLoad>(kp + o.koff[st] + i * 64);
#pragma unroll
  for (int nc = 0; nc < S::NC; ++nc) R.v[nc] = load_stream<VLoad>(vp + o.voff + nc * vstride);
}

// Page k of range wr (its loads in R): S^T = K q^T per head tile, online
// softmax, O^T += V^T P^T, for the lane's item state (q operands qop, q
// channel sum qsum for the zero-point term, running max m, sum lsum,
// zero-point sum zacc, accumulators acc, V-scale exponent vexp).  Absent
// pages are skipped; on a partial page (some token past the sequence or
// outside the window) those tokens' scores are -inf and their V^T values (or
// V scales) 0.
//
// Quantized pools: a token's P.V operand is its weight times its V scale,
// rounded to float16.  Small V scales would put it among float16's
// subnormals, large ones (FP8 codes carry 2^8) past its range, so the
// weights carry a power of two 2^c: vexp is the largest (biased float32)
// exponent of a V scale the item has seen and c = vexp_offset(vexp), which
// keeps every operand below 2^15.  lsum, zacc and acc are all in units of
// 2^c (their ratio, the output, does not depend on it); when a page raises
// vexp, c drops and the running sums are rescaled with the softmax factor.
struct PageVInRegs {};  // mfma_page's default: the V^T bytes are in R.v
template <int F, int P, int D, int NT, typename VFetch = PageVInRegs>
__device__ __forceinline__ void mfma_page(const DecodeArgs& a, const PageRegs<F, P, D>& R,
                                          const WorkRange& wr, int k, int r, int gq,
                                          const typename MfmaOps<F, P, D>::A (&qop)[NT][MfmaShape<F, P, D>::KK],
                                          const float (&qsum)[NT], float (&m)[NT], float (&lsum)[NT],
                                          float (&zacc)[NT], f32x4_t (&acc)[NT][MfmaShape<F, P, D>::NC],
                                          int& vexp, const VFetch& vfetch = VFetch{}) {
  using S = MfmaShape<F, P, D>;
  using FI = FmtInfo<F>;
  constexpr bool Q = FI::quant, ZP = FI::zero;
  constexpr int T = S::T, KK = S::KK, NC = S::NC, EV = S::EV, KB = S::KB;
  using OpA = typename MfmaOps<F, P, D>::A;
  using OpPV = typename MfmaOps<F, P, D>::PV;
  using VLoad = typename LoadT<S::VB>::type;

  if (R.phys < 0) return;  // absent page: its tokens do not take part
  const PageMask pm = page_mask<P>(wr, wr.logical(wr.kb0 + k));
  const bool tail = pm.partial;

  // K operands for all sub-tiles (shared by every head tile).
  OpA kop[T][KK];
#pragma unroll
  for (int st = 0; st < T; ++st) {
    if constexpr (!Q) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kop[st][kk] = __builtin_bit_cast(bf16x8_t, R.k[st][kk]);
    } else {
      uint32_t w[KB / 4];
      __builtin_memcpy(w, R.k[st], KB);
      constexpr int DW = F == kI4 ? 1 : 2;  // dwords per 8 channels
      // INT4: the float16 exponent bits in a register (an empty asm hides
      // the constant), so that each mask-and-or is one instruction (it cannot
      // take two literal constants): 16 sequences of 16k-32k tokens, 93.8 ->
      // 92.9 us for the decode call
      uint32_t expo = 0x64006400u;
      if constexpr (F == kI4) asm("" : "+v"(expo));
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kop[st][kk] = codes8_to_f16x8_offset<F>(w + DW * kk, expo);
    }
  }
  // V^T operands: from R.v, or (late_v) from vfetch right before P.V, so
  // that the V^T bytes do not hold registers while the scores are computed
  constexpr bool late_v = !std::is_same<VFetch, PageVInRegs>::value;
  OpPV vop[NC];
  auto build_vop = [&](const VLoad (&vraw)[NC]) __attribute__((always_inline)) {
#pragma unroll
  for (int nc = 0; nc < NC; ++nc) {
    if constexpr (!Q) {
      VLoad raw = vraw[nc];
      if (tail) {
        // rows past the sequence may hold anything (NaN): zero them so 0*x stays 0
        uint32_t wv[EV / 2];
        __builtin_memcpy(wv, &raw, sizeof(raw));
#pragma unroll
        for (int e = 0; e < EV; ++e) {
          if (!pm.valid(EV * gq + e)) wv[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
        __builtin_memcpy(&raw, wv, sizeof(raw));
      }
      vop[nc] = __builtin_bit_cast(OpPV, raw);
    } else {
      uint32_t wv[EV / 4];
      __builtin_memcpy(wv, &vraw[nc], sizeof(vraw[nc]));
      OpPV v;
#pragma unroll
      for (int i = 0; i < EV / 4; ++i) {
        f16x2_t lo, hi;
        codes4_to_f16x4<F>(wv[i], (r & 1) != 0, lo, hi);
        v[4 * i + 0] = lo[0];
        v[4 * i + 1] = lo[1];
        v[4 * i + 2] = hi[0];
        v[4 * i + 3] = hi[1];
      }
      vop[nc] = v;
    }
  }
  };
  if constexpr (!late_v) build_vop(R.v);
  // Per-token scale (and zero point) of this lane's rows.  The V metadata of
  // tokens not kept may hold anything (NaN): it is zeroed, so that their zero
  // weights give exact zeros below.
  float ks[T][4], kz[T][4], vs[T][4], vz[T][4];
  if constexpr (Q) {
#pragma unroll
    for (int st = 0; st < T; ++st) {
      const uint32_t kw[4] = {R.km[st].x, R.km[st].y, R.km[st].z, R.km[st].w};
      uint32_t vw[4] = {R.vm[st].x, R.vm[st].y, R.vm[st].z, R.vm[st].w};
      if (tail) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!pm.valid(EV * gq + 4 * st + i)) vw[i] = 0u;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ks[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(kw[i] & 0xffffu)) * FI::scale_mul;
        kz[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(kw[i] >> 16));
        vs[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(vw[i] & 0xffffu)) * FI::scale_mul;
        vz[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(vw[i] >> 16));
      }
    }
  }
  // the offset c, raised only when some V scale of the page (tokens not kept
  // have 0) has a larger exponent than any before in the item (wave-uniform)
  int cnew = vexp_offset(vexp), cdelta = 0;
  if constexpr (Q) {
    float vmax = 0.0f;
#pragma unroll
    for (int st = 0; st < T; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) vmax = fmaxf(vmax, vs[st][i]);
    if (wave_any(__float_as_uint(vmax) >= uint32_t(vexp + 1) << 23)) {
      vmax = group4_max(vmax);
      const int e = __builtin_amdgcn_readfirstlane(int(__float_as_uint(vmax) >> 23));
      const int cold = cnew;
      vexp = max(vexp, e);
      cnew = vexp_offset(vexp);
      cdelta = cnew - cold;
    }
  }
  // scores are cs times a raw dot product; the multiply rides in the
  // exponent's fma (cs > 0 keeps masked scores at -inf)
  const float cs = fmaxf(fabsf(a.scale_log2), 1e-30f);

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float x[T][4];
#pragma unroll
    for (int st = 0; st < T; ++st) {
      f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (FI::koff != 0.0f) {
        // sum over channels of q (code + koff), minus koff sum(q): q . code
        const float c0 = -FI::koff * qsum[nt];
        sc = f32x4_t{c0, c0, c0, c0};
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sc = mfma_16x16x32(kop[st][kk], qop[nt][kk], sc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (ZP)
          x[st][i] = ks[st][i] * sc[i] + kz[st][i] * qsum[nt];
        else if constexpr (Q)
          x[st][i] = ks[st][i] * sc[i];
        else
          x[st][i] = sc[i];
      }
    }
    if (tail) {
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!pm.valid(EV * gq + 4 * st + i)) x[st][i] = -INFINITY;
    }
    float mloc = x[0][0];
#pragma unroll
    for (int st = 0; st < T; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, x[st][i]);
    mloc = group4_max(mloc);
    // m: the running maximum of the scaled scores (base-2 units)
    const float mnew = fmaxf(m[nt], mloc * cs);
    const float al = fast_exp2(Q ? (m[nt] - mnew) + float(cdelta) : m[nt] - mnew);
    m[nt] = mnew;
    // weights 2^(score - m + c)
    const float mref = Q ? mnew - float(cnew) : mnew;
    float p[T][4];
    float ps = 0.0f;
#pragma unroll
    for (int st = 0; st < T; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[st][i] = fast_exp2(fmaf(x[st][i], cs, -mref));
        ps += p[st][i];
      }
    lsum[nt] = lsum[nt] * al + ps;
    // once the running maximum settles, al is exactly 1 for every head:
    // skip the (identity) rescale of the accumulators
    if (wave_any(al != 1.0f)) {
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) acc[nt][nc] *= al;
    }
    OpPV pop;
    if constexpr (Q) {
      float zs = 0.0f;
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // (a token not kept has weight 0 and zeroed V metadata); slot i
          // holds token kV4Slot(i), the V^T operand's order
          const int t = kV4Slot<F>(i);
          const float pv = p[st][t] * vs[st][t];
          if constexpr (ZP) zs += p[st][t] * vz[st][t];
          pop[4 * st + i] = (_Float16)pv;
        }
      zacc[nt] = zacc[nt] * al + zs;
    } else {
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) pop[4 * st + i] = (__bf16)p[st][i];
    }
    if constexpr (late_v) {
      if (nt == 0) {
        VLoad vraw[NC];
        vfetch(vraw);
        build_vop(vraw);
      }
    }
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) {
      if constexpr (T == 1)
        acc[nt][nc] = mfma_16x16x16(vop[nc], pop, acc[nt][nc]);
      else
        acc[nt][nc] = mfma_16x16x32(vop[nc], pop, acc[nt][nc]);
    }
  }
  }

template <int F, int P, int D, int NT, int DEPTH, bool SCHED>
__device__ __forceinline__ void mfma_item(const DecodeArgs& a, const WorkRange& wr, float* smem) {
  using S = MfmaShape<F, P, D>;
  using FI = FmtInfo<F>;
  constexpr bool ZP = FI::zero;
  constexpr int KK = S::KK, NC = S::NC;
  constexpr int HP = NT * 16;
  using OpA = typename MfmaOps<F, P, D>::A;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int g = a.group;

  // q^T as the B operand of S^T = K q^T
  OpA qop[NT][KK];
  float qsum[NT];
  mfma_load_q<F, P, D, NT>(a, wr.b, wr.h, r, gq, qop, qsum);

  const int32_t* btrow = a.bt + int64_t(wr.b) * a.max_blocks;

  const MfmaLaneOffsets<F, P, D> lo = mfma_lane_offsets<F, P, D>(r, gq);
  auto issue = [&](PageRegs<F, P, D>& R, int k) {
    mfma_load_page<F, P, D>(a, btrow[wr.logical(wr.kb0 + k)], wr.h, lo, R);
  };

  float m[NT], lsum[NT], zacc[NT];
  f32x4_t acc[NT][NC];
  int vexp = 0;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    lsum[nt] = 0.0f;
    zacc[nt] = 0.0f;
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) acc[nt][nc] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  auto compute = [&](const PageRegs<F, P, D>& R, int k) {
    mfma_page<F, P, D, NT>(a, R, wr, k, r, gq, qop, qsum, m, lsum, zacc, acc, vexp);
  };
  if (wr.cnt > 0) {
    PageRegs<F, P, D> ring[DEPTH];
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) issue(ring[s], min(s, wr.cnt - 1));
    for (int k0 = 0; k0 < wr.cnt; k0 += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        const int k = k0 + s;
        if (k < wr.cnt) compute(ring[s], k);
        // always refill (clamped to the last page: a cache hit, no HBM traffic)
        // so the in-order load counter stays a compile-time pattern
        issue(ring[s], min(k + DEPTH, wr.cnt - 1));
      }
    }
  }

  // Wavefront partials -> LDS, in plain units (each wavefront has its own 2^c).
  float* sm_o = smem;                 // [W][g][D]
  float* sm_m = smem + W * g * D;     // [W][HP]
  float* sm_l = sm_m + W * HP;        // [W][HP]
  const float unc = exp2_int(-vexp_offset(vexp));
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = group4_sum(lsum[nt]) * unc;
    const float zt = ZP ? group4_sum(zacc[nt]) : 0.0f;
    const int jj = nt * 16 + r;
    if (jj < g) {
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) {
        f32x4_t v = acc[nt][nc];
        if constexpr (ZP) v += zt;
        v *= unc;
        *reinterpret_cast<f32x4_t*>(sm_o + (wave * g + jj) * D + 16 * nc + 4 * gq) = v;
      }
      if (gq == 0) {
        sm_m[wave * HP + jj] = m[nt];
        sm_l[wave * HP + jj] = lt;
      }
    }
  }
  __syncthreads();
  combine_and_store<D, SCHED>(a, wr, sm_o, sm_m, sm_l, W, HP);
}

// One workgroup: a (sequence, KV head, split) of the uniform plan.
template <int F, int P, int D, int NT, int DEPTH>
__global__ __launch_bounds__(mfma_max_threads(P, D, NT)) void decode_mfma_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  mfma_item<F, P, D, NT, DEPTH, false>(a, work_range<P>(a, wave, W), smem);
}

// ---------------------------------------------------------------------------
// Balanced schedule on the matrix-core path: one wavefront streams one bin.
// The bin's items (pieces of (sequence, KV head) pairs) pass through the
// same register ring one after another, so the loads of an item's first
// pages are in flight while the previous item's last pages are computed, and
// no workgroup barrier separates items: the wavefront writes each item's
// result (the output, or a normalized partial for the merge) from its own
// registers.  Wavefronts of a workgroup are independent.

// Where one side (issue or compute) of a stream stands: item `item` of the
// schedule (== end once the stream is done), page k of its range.
struct StreamPos {
  int item, k;
  WorkRange wr;
};

// From p.item on: the first valid item (with nonempty range when
// need_pages), its range loaded and k = 0.
template <int P>
__device__ __forceinline__ void stream_seek(const DecodeArgs& a, StreamPos& p, int end,
                                            bool need_pages) {
  for (; p.item < end; ++p.item) {
    if (!item_valid(a, p.item)) continue;
    p.wr = item_range<P>(a, p.item, 0, 1);
    if (!need_pages || p.wr.cnt > 0) break;
  }
  p.k = 0;
}

// Wavefronts per SIMD the stream kernel is compiled for.  Quantized pages
// carry much more arithmetic per byte than bfloat16 ones (code conversion,
// scales, zero points), and with several wavefronts per SIMD one computes
// while the others wait on memory.  Measured on 16 sequences of 16k-32k
// tokens, P = 32: INT8 176 -> 166 us and FP8 159 -> 150 us with two (and
// one-page rings: two-page rings spill and were slower; three wavefronts
// measured 2-6% slower); INT4, whose pages are half the bytes, 166 -> 142 us
// with two and two-page rings, and 139 -> 121 us from there with three
// wavefronts and one-page rings (168 registers, no spills).  bfloat16 keeps
// one wavefront with a two-page ring (two measured slower).  Only instances
// for groups of up to 16 query heads (one head tile) fit those register
// budgets; larger groups keep one wavefront.
template <int F, int NT> constexpr int stream_waves_per_simd() {
  return F == kBF16 || NT != 1 ? 1 : (F == kI4 ? 3 : 2);
}

// LDS page ring.  A wavefront's page loads are bounded by the registers they
// land in: three INT4 wavefronts per SIMD with one page each keep about 13 MB
// in flight on the chip, and at the loaded latency that sustains ~4.5 TB/s.
// The loads can land in LDS instead (global_load_lds: each lane's 4 or 16
// bytes go to the LDS base in m0 plus lane * size), where a wavefront keeps
// several pages in flight for no registers; the page being computed is read
// from its slot into the same registers the register ring would hold.  Used
// by the stream kernel for INT4 pools with 32-token pages of 128 channels
// (one head tile): 16 sequences of 16k-32k tokens measured 100.5 -> 96.4 us
// for the whole decode call, and 94.6 with the K codes' offset left in (the
// ring moved the limit to the vector ALUs).  The same ring measured 3-5%
// slower for INT8, FP8 (two wavefronts per SIMD, two slots) and bfloat16
// (one wavefront per SIMD, four slots): fewer wavefronts leave the slot
// reads' latency exposed.
template <int F, int P, int D, int NT> constexpr bool stream_lds_ring() {
  return F == kI4 && P == 32 && D == 128 && NT == 1;
}
template <int F, int P, int D> struct LdsSlot {
  static constexpr int TB = P * MfmaShape<F, P, D>::RB;     // one K (or V) tile
  static constexpr int MB = FmtInfo<F>::quant ? P * 4 : 0;  // its (scale, zero) pairs
  static constexpr int SB = 2 * TB + 2 * MB;                // K, V, K meta, V meta
  // pages in flight per wavefront: the slots of a compute unit's twelve
  // INT4 wavefronts (three per SIMD) fill 153 of its 160 KiB of LDS
  static constexpr int depth = 3;
  static constexpr int k_loads = TB / 1024, v_loads = TB / 1024;
  static constexpr int loads = (MB ? 1 : 0) + k_loads + v_loads;  // copies per page
};
// One copy instruction: `bytes` (4 or 16) per lane from the lane's global
// address to LDS byte m0 + lane * bytes, with the streaming cache policy
// (page data) or the default one (`cached`).
// The copies and the slot reads below are asm statements that are not
// volatile (the compiler treats its own LDS-copy builtin, and any volatile
// asm, as writing all memory, and would then read the read-only tables with
// vector loads, whose waits wait for every copy in flight); they are kept in
// program order by one token that each takes and passes on ("+s"), and the
// last wait takes it too.  The compiler does not count these copies in its
// own load-counter waits, which only makes those waits longer (the counter
// retires loads in order); the slot reads wait for them explicitly.  (An SALU
// write of m0 needs one wait state before a copy reads it.)
template <int bytes, bool cached = false>
__device__ __forceinline__ void lds_copy(const void* src, uint32_t lds_addr, uint32_t& tok) {
  static_assert(bytes == 4 || bytes == 16, "dword or dwordx4 copies");
  if constexpr (cached) {
    static_assert(bytes == 4, "cached copies are the ring's 4-byte fillers");
    asm("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off"
        : "+s"(tok)
        : "s"(lds_addr), "v"(src)
        : "m0");
  } else if constexpr (bytes == 16)
    asm("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off nt"
        : "+s"(tok)
        : "s"(lds_addr), "v"(src)
        : "m0");
  else
    asm("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off nt"
        : "+s"(tok)
        : "s"(lds_addr), "v"(src)
        : "m0");
}

// Copy one (page, head) tile into an LDS slot as flat byte ranges (lane l's
// bytes at l * size): both metadata rows (K's 128 bytes, then V's), the K
// tile, the V^T tile.  Out of range table entries read page 0 (the pattern
// stays fixed) and return -1.
template <int F, int P, int D>
__device__ __forceinline__ int lds_load_page(const DecodeArgs& a, int phys, int h, int lane,
                                             uint32_t slot, uint32_t& tok) {
  using L = LdsSlot<F, P, D>;
  static_assert(L::TB % 1024 == 0 && (L::MB == 0 || L::MB == 128),
                "1 KiB copies and one metadata row");
  const bool ok = unsigned(phys) < unsigned(a.num_pages);
  const int64_t tile = int64_t(ok ? phys : 0) * a.num_kv_heads + h;
  if constexpr (L::MB > 0) {
    const char* km = reinterpret_cast<const char*>(a.k_meta) + tile * L::MB;
    const char* vm = reinterpret_cast<const char*>(a.v_meta) + tile * L::MB;
    const char* mp = lane < 32 ? km + 4 * lane : vm + 4 * (lane - 32);
    lds_copy<4>(mp, slot + 2 * L::TB, tok);
  }
  const char* kp = static_cast<const char*>(a.k_pool) + tile * L::TB + 16 * lane;
  const char* vp = static_cast<const char*>(a.v_pool) + tile * L::TB + 16 * lane;
#pragma unroll
  for (int i = 0; i < L::k_loads; ++i) lds_copy<16>(kp + 1024 * i, slot + 1024 * i, tok);
#pragma unroll
  for (int i = 0; i < L::v_loads; ++i)
    lds_copy<16>(vp + 1024 * i, slot + L::TB + 1024 * i, tok);
  return ok ? phys : -1;
}

// The ring's filler once a stream's pages are all issued: as many copy
// instructions as a page (the slot reads' waits count them), each of 256
// bytes that stay cached (the first q row, 4 bytes per lane), into a slot
// that is never read again.  Re-issuing the last page instead, as the
// register ring does, re-read it from HBM: three fillers per bin added 3% to
// INT4's traffic.
template <int F, int P, int D>
__device__ __forceinline__ void lds_load_filler(const DecodeArgs& a, int lane, uint32_t slot,
                                                uint32_t& tok) {
  static_assert(D == 128 && LdsSlot<F, P, D>::loads * 256 <= LdsSlot<F, P, D>::SB,
                "a 256-byte q row, copies within the slot");
  const char* src = reinterpret_cast<const char*>(a.q) + 4 * lane;
#pragma unroll
  for (int i = 0; i < LdsSlot<F, P, D>::loads; ++i) lds_copy<4, true>(src, slot + 256 * i, tok);
}

// Read a slot into a lane's page registers (the register ring's layout), in
// two parts: K and the metadata when the page is computed, V^T right before
// its P.V products.  Each part first waits until its copies have landed:
// `later` copy instructions were issued after them (any other memory
// operation issued since only makes the wait longer); its reads and both
// waits sit in one asm block, so no read is in flight when it ends.  Lane
// addresses: ak = the lane's first K piece, am = its metadata, av = its V^T
// bytes; the offsets in the reads follow the register ring's loads
// (mfma_load_page) for each shape.
template <int F, int P, int D> struct LdsRead;
// INT4, 32-token pages: K sub-tile 1 is four token rows (256 bytes) past
// sub-tile 0; V^T chunk nc at nc * 8P = 256 bytes (read2 offsets count 8
// bytes); metadata: K's rows at 0 and 16, V's 128 bytes later.
template <> struct LdsRead<kI4, 32, 128> {
  using S = MfmaShape<kI4, 32, 128>;
  static_assert(S::T == 2 && S::KN == 1 && S::NC == 8 && S::VB == 8 && S::RB == 64,
                "32-token INT4 pages of 128 channels");
  template <int later>
  __device__ static void k_meta(uint32_t ak, uint32_t am, PageRegs<kI4, 32, 128>& R,
                                uint32_t& tok) {
    asm("s_waitcnt vmcnt(%[later])\n\t"
        "ds_read_b128 %[k0], %[ak]\n\t"
        "ds_read_b128 %[k1], %[ak] offset:256\n\t"
        "ds_read_b128 %[km0], %[am]\n\t"
        "ds_read_b128 %[km1], %[am] offset:16\n\t"
        "ds_read_b128 %[vm0], %[am] offset:128\n\t"
        "ds_read_b128 %[vm1], %[am] offset:144\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [k0] "=&v"(R.k[0][0]), [k1] "=&v"(R.k[1][0]), [km0] "=&v"(R.km[0]),
          [km1] "=&v"(R.km[1]), [vm0] "=&v"(R.vm[0]), [vm1] "=&v"(R.vm[1]), [tok] "+s"(tok)
        : [ak] "v"(ak), [am] "v"(am), [later] "n"(later));
  }
  template <int later>
  __device__ static void v(uint32_t av, uint2 (&v)[8], uint32_t& tok) {
    uint4 v01, v23, v45, v67;
    asm("s_waitcnt vmcnt(%[later])\n\t"
        "ds_read2_b64 %[v01], %[av] offset1:32\n\t"
        "ds_read2_b64 %[v23], %[av] offset0:64 offset1:96\n\t"
        "ds_read2_b64 %[v45], %[av] offset0:128 offset1:160\n\t"
        "ds_read2_b64 %[v67], %[av] offset0:192 offset1:224\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [v01] "=&v"(v01), [v23] "=&v"(v23), [v45] "=&v"(v45), [v67] "=&v"(v67),
          [tok] "+s"(tok)
        : [av] "v"(av), [later] "n"(later));
    v[0] = make_uint2(v01.x, v01.y);
    v[1] = make_uint2(v01.z, v01.w);
    v[2] = make_uint2(v23.x, v23.y);
    v[3] = make_uint2(v23.z, v23.w);
    v[4] = make_uint2(v45.x, v45.y);
    v[5] = make_uint2(v45.z, v45.w);
    v[6] = make_uint2(v67.x, v67.y);
    v[7] = make_uint2(v67.z, v67.w);
  }
};
template <int F, int P, int D, int NT, int DEPTH>
__global__ __launch_bounds__(256, (stream_waves_per_simd<F, NT>())) void decode_mfma_stream_kernel(
    DecodeArgs a) {
  using S = MfmaShape<F, P, D>;
  using FI = FmtInfo<F>;
  constexpr bool ZP = FI::zero;
  constexpr int KK = S::KK, NC = S::NC;
  using OpA = typename MfmaOps<F, P, D>::A;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bin = blockIdx.x * (blockDim.x >> 6) + wave;
  if (bin >= a.num_bins) return;  // the whole wavefront; nothing here waits on the others
  const int r = lane & 15, gq = lane >> 4;
  const int g = a.group;
  const int i_begin = max(a.sched[8 + bin], 0);
  const int end = min(a.sched[9 + bin], a.num_items);

  // issue side: loads page ip.k of item ip.item; once the stream's pages are
  // all issued it repeats the last page (a cache hit) so the ring's load
  // pattern stays fixed
  StreamPos ip;
  ip.item = i_begin;
  stream_seek<P>(a, ip, end, true);
  bool issued_all = ip.item >= end;
  const MfmaLaneOffsets<F, P, D> lo = mfma_lane_offsets<F, P, D>(r, gq);
  // the ring: RD pages in registers, or (LR) in this wavefront's LDS slots
  // with only their page ids in registers
  constexpr bool LR = stream_lds_ring<F, P, D, NT>();
  using LS = LdsSlot<F, P, D>;
  constexpr int RD = LR ? LS::depth : DEPTH;
  __shared__ __attribute__((aligned(16))) char lds_ring[LR ? 4 * RD * LS::SB : 16];
  // this wavefront's slots (an LDS byte address: the low half of the generic one)
  const uint32_t wslots =
      uint32_t(reinterpret_cast<uintptr_t>(lds_ring)) + (LR ? wave * RD * LS::SB : 0);
  PageRegs<F, P, D> ring[LR ? 1 : RD];
  int ring_phys[RD];
  uint32_t ltok = 0;  // orders the LDS ring's asm statements
  auto issue = [&](int s) __attribute__((always_inline)) {
    const int32_t* btrow = a.bt + int64_t(ip.wr.b) * a.max_blocks;
    const int phys = btrow[ip.wr.logical(ip.wr.kb0 + ip.k)];
    if constexpr (LR) {
      if (issued_all)  // every page is issued: a filler keeps the count of copies
        lds_load_filler<F, P, D>(a, lane, wslots + s * LS::SB, ltok);
      else
        ring_phys[s] = lds_load_page<F, P, D>(a, phys, ip.wr.h, lane, wslots + s * LS::SB, ltok);
    } else
      mfma_load_page<F, P, D>(a, phys, ip.wr.h, lo, ring[s]);
    // advance to the next page of the stream (or stay on the last one)
    if (!issued_all) {
      if (++ip.k >= ip.wr.cnt) {
        StreamPos nx = ip;
        ++nx.item;
        stream_seek<P>(a, nx, end, true);
        if (nx.item < end) ip = nx;
        else { issued_all = true; ip.k = ip.wr.cnt - 1; }
      }
    }
  };

  // per-item state: q operands, online softmax
  OpA qop[NT][KK];
  float qsum[NT];
  float m[NT], lsum[NT], zacc[NT];
  f32x4_t acc[NT][NC];
  int vexp = 0;
  // One head tile (NT = 1, and two wavefronts per SIMD at most: INT4's three
  // have no registers to spare): the next item with pages has its q loaded
  // while the current one is computed, so an item's first page does not wait
  // on the q loads issued behind the ring's pages.
  constexpr bool QPRE = NT == 1 && stream_waves_per_simd<F, NT>() <= 2;
  uint4 qnext[NT][KK];
  auto prefetch_q = [&](int from) __attribute__((always_inline)) {
    StreamPos qp;
    qp.item = from;
    stream_seek<P>(a, qp, end, true);
    if (qp.item < end) mfma_q_raw<F, P, D, NT>(a, qp.wr.b, qp.wr.h, r, gq, qnext);
  };
  auto begin_item = [&](const WorkRange& wr, int item) __attribute__((always_inline)) {
    if constexpr (QPRE) {
      // items with pages come in the same order as the prefetches
      if (wr.cnt > 0) {
        mfma_q_convert<F, P, D, NT>(a, qnext, qop, qsum);
        prefetch_q(item + 1);
      }
    } else {
      mfma_load_q<F, P, D, NT>(a, wr.b, wr.h, r, gq, qop, qsum);
    }
    vexp = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m[nt] = -INFINITY;
      lsum[nt] = 0.0f;
      zacc[nt] = 0.0f;
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) acc[nt][nc] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  // the item's result: o / l (and m, l for a partial), straight from registers
  auto finish_item = [&](const WorkRange& wr) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float lt = group4_sum(lsum[nt]);
      const float zt = ZP ? group4_sum(zacc[nt]) : 0.0f;
      const int jj = nt * 16 + r;
      if (jj < g) {
        const int64_t row = int64_t(wr.b) * a.num_q_heads + int64_t(wr.h) * g + jj;
        const int64_t pr = int64_t(wr.slot) * g + jj;
        // one reciprocal per head (o * (1/l): within an ulp of o / l in float32)
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) {
          f32x4_t v = acc[nt][nc];
          if constexpr (ZP) v += zt;
          v *= inv;
          const int d = 16 * nc + 4 * gq;
          if (wr.slot < 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a.out[row * D + d + i] = f32_to_bf16_rne(v[i]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) a.part_o[pr * D + d + i] = v[i];
          }
        }
        if (wr.slot >= 0 && gq == 0) {
          a.part_ml[pr * 2] = m[nt];
          a.part_ml[pr * 2 + 1] = lt * exp2_int(-vexp_offset(vexp));  // plain units
        }
      }
    }
  };

  // lane addresses of the LDS slots' pieces (slot 0; slot s is s * SB on)
  uint32_t lds_k = 0, lds_v = 0, lds_m = 0;
  if constexpr (LR) {
    lds_k = wslots + lo.koff[0];
    lds_v = wslots + LS::TB + lo.voff;
    lds_m = wslots + 2 * LS::TB + lo.moff;
  }
  auto compute = [&](int s, const WorkRange& wr, int k) __attribute__((always_inline)) {
    if constexpr (LR) {
      // the pages issued after this one are later copies still in flight;
      // this page's own V^T copies come after its K and metadata ones
      constexpr int later = (RD - 1) * LS::loads;
      static_assert(later + LS::v_loads <= 63, "load counter range");
      PageRegs<F, P, D> R;
      LdsRead<F, P, D>::template k_meta<later + LS::v_loads>(lds_k + s * LS::SB,
                                                              lds_m + s * LS::SB, R, ltok);
      R.phys = ring_phys[s];
      const uint32_t av = lds_v + s * LS::SB;
      auto vfetch = [av, &ltok](uint2 (&v)[8]) __attribute__((always_inline)) {
        LdsRead<F, P, D>::template v<later>(av, v, ltok);
      };
      mfma_page<F, P, D, NT>(a, R, wr, k, r, gq, qop, qsum, m, lsum, zacc, acc, vexp, vfetch);
    } else {
      mfma_page<F, P, D, NT>(a, ring[s], wr, k, r, gq, qop, qsum, m, lsum, zacc, acc, vexp);
    }
  };

  // compute side: every valid item in order (empty ones give 0 or an empty
  // partial right away); pages in the order they were issued.  Each item's
  // pages run through a loop whose ring slots are compile-time constants
  // (like the uniform kernel's), so the load counter waits stay those of a
  // steady stream; the item's start and end (q loads, result stores) sit
  // outside that loop.
  static_assert(RD >= 1 && RD <= 4, "stream ring of one to four pages");
  StreamPos cp;
  cp.item = i_begin;
  stream_seek<P>(a, cp, end, false);
  if (issued_all) {  // no pages at all: only empty items
    for (; cp.item < end; ++cp.item, stream_seek<P>(a, cp, end, false)) {
      begin_item(cp.wr, cp.item);
      finish_item(cp.wr);
    }
    return;
  }
  if constexpr (QPRE) prefetch_q(cp.item);
#pragma unroll
  for (int s = 0; s < RD; ++s) issue(s);
  // pages of the current item, its first page in ring slot S0
  auto item_pages = [&](auto s0_tag) __attribute__((always_inline)) {
    constexpr int S0 = decltype(s0_tag)::value;
    const int cnt = cp.wr.cnt;
    int k = 0;
    for (; k + RD <= cnt; k += RD) {
#pragma unroll
      for (int s = 0; s < RD; ++s) {
        compute((S0 + s) % RD, cp.wr, k + s);
        issue((S0 + s) % RD);
      }
    }
    // fewer than RD pages left, from slot S0 on
#pragma unroll
    for (int s = 0; s < RD - 1; ++s) {
      if (k + s < cnt) {
        compute((S0 + s) % RD, cp.wr, k + s);
        issue((S0 + s) % RD);
      }
    }
  };
  auto pages_from_slot = [&](int s0) __attribute__((always_inline)) {
    if (s0 == 0) {
      item_pages(std::integral_constant<int, 0>{});
    } else if constexpr (RD > 1) {
      if (s0 == 1) {
        item_pages(std::integral_constant<int, 1>{});
      } else if constexpr (RD > 2) {
        if (s0 == 2)
          item_pages(std::integral_constant<int, 2>{});
        else if constexpr (RD > 3)
          item_pages(std::integral_constant<int, 3>{});
      }
    }
  };
  int slot0 = 0;
  for (; cp.item < end; ++cp.item, stream_seek<P>(a, cp, end, false)) {
    begin_item(cp.wr, cp.item);
    if (cp.wr.cnt > 0) {
      pages_from_slot(slot0);
      slot0 = (slot0 + cp.wr.cnt) % RD;
    }
    finish_item(cp.wr);
  }
  // the ring's last copies land before the wavefront (and its LDS) ends
  if constexpr (LR) asm volatile("s_waitcnt vmcnt(0) ; %0" : : "s"(ltok));
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel for g < 4.  Lane l: token row tr = l/4 (+16 per extra
// sub-tile), channel quarter c = l%4 for q.k; output channels l*D/64.. for P.V.
template <int F>
__device__ __forceinline__ float code_to_f32(uint32_t byte_or_nibble) {
  if constexpr (F == kI8) {
    return float(int8_t(byte_or_nibble & 0xffu));
  } else if constexpr (F == kI4) {
    return float(int(byte_or_nibble & 0xfu) - 8);
  } else {  // e4m3 value times 2^-8 (the scale carries 2^8)
    const uint32_t b = byte_or_nibble & 0xffu;
    return (float)__builtin_bit_cast(_Float16, uint16_t(((b & 0x80u) << 8) | ((b & 0x7fu) << 7)));
  }
}

template <int F, int P, int D, int G, int DEPTH, bool SCHED>
__device__ __forceinline__ void valu_item(const DecodeArgs& a, const WorkRange& wr, float* smem) {
  using FI = FmtInfo<F>;
  constexpr bool Q = FI::quant, ZP = FI::zero;
  constexpr int TPL = P / 16;             // token rows per lane
  constexpr int DQ = D / 4;               // channels per lane for q.k
  constexpr int DV = D / 64;              // output channels per lane
  constexpr int RB = D * FI::bits / 8;    // bytes of a stored token row
  constexpr int KB = DQ * FI::bits / 8;   // K bytes per lane per token row
  constexpr int KLB = KB >= 16 ? 16 : KB;
  constexpr int KN = KB / KLB;
  // V^T bytes per lane: its DV channels over P tokens ([D][P] elements; for
  // INT4 the P bytes of the channel pair holding them)
  constexpr int VBT = F == kI4 ? P : DV * P * FI::bits / 8;
  constexpr int VL = VBT / 16;
  using KLoad = typename LoadT<KLB>::type;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int tr = lane >> 2, c = lane & 3;
  const int H = a.num_kv_heads;
  float* sm_o = smem;                  // [W][G][D]
  float* sm_m = smem + W * G * D;      // [W][G]
  float* sm_l = sm_m + W * G;          // [W][G]
  float* pbuf = sm_l + W * G + wave * G * P;  // this wave's [G][P] probabilities

  float qf[G][DQ];
  float qsum[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint16_t* qrow = a.q + (int64_t(wr.b) * a.num_q_heads + int64_t(wr.h) * G + j) * D;
    float qs = 0.0f;
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      qf[j][e] = bf16_to_f32(qrow[c * DQ + e]);
      qs += qf[j][e];
    }
    qs += __shfl_xor(qs, 1);
    qs += __shfl_xor(qs, 2);
    qsum[j] = qs;
  }

  struct Regs {
    KLoad k[TPL][KN];
    uint4 v[VL];
    uint32_t km[TPL], vm[TPL];
    int phys;
  };
  const size_t tile_bytes = size_t(P) * RB;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int32_t* btrow = a.bt + int64_t(wr.b) * a.max_blocks;
  const int vrow = F == kI4 ? (DV == 2 ? lane : (lane >> 1)) * P : lane * VBT;

  auto issue = [&](Regs& R, int k) {
    int phys = btrow[wr.logical(wr.kb0 + k)];
    const bool ok = unsigned(phys) < unsigned(a.num_pages);
    R.phys = ok ? phys : -1;
    const int64_t tile = int64_t(ok ? phys : 0) * H + wr.h;
    const char* kp = kbase + tile * tile_bytes;
    const char* vp = vbase + tile * tile_bytes;
#pragma unroll
    for (int u = 0; u < TPL; ++u)
#pragma unroll
      for (int i = 0; i < KN; ++i)
        R.k[u][i] = load_stream<KLoad>(kp + (tr + 16 * u) * RB + c * KB + KLB * i);
#pragma unroll
    for (int i = 0; i < VL; ++i) R.v[i] = load_stream<uint4>(vp + vrow + 16 * i);
    if constexpr (Q) {
      const uint32_t* km = reinterpret_cast<const uint32_t*>(a.k_meta) + tile * P;
      const uint32_t* vm = reinterpret_cast<const uint32_t*>(a.v_meta) + tile * P;
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        R.km[u] = load_stream<uint32_t>(km + tr + 16 * u);
        R.vm[u] = load_stream<uint32_t>(vm + tr + 16 * u);
      }
    }
  };

  float m[G], lsum[G], zacc[G], acc[G][DV];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    lsum[j] = 0.0f;
    zacc[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < DV; ++e) acc[j][e] = 0.0f;
  }

  auto compute = [&](const Regs& R, int k) {
    if (R.phys < 0) return;
    const PageMask pm = page_mask<P>(wr, wr.logical(wr.kb0 + k));
    const bool tail = pm.partial;
    float x[TPL][G];
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
      float kv[DQ];
      uint32_t w[KB / 4];
      __builtin_memcpy(w, R.k[u], KB);
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        if constexpr (F == kBF16)
          kv[e] = bf16_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
        else if constexpr (F == kI4)
          kv[e] = code_to_f32<F>(w[e >> 3] >> (4 * (e & 7)));
        else
          kv[e] = code_to_f32<F>(w[e >> 2] >> (8 * (e & 3)));
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float dsum = 0.0f;
#pragma unroll
        for (int e = 0; e < DQ; ++e) dsum += qf[j][e] * kv[e];
        dsum += __shfl_xor(dsum, 1);
        dsum += __shfl_xor(dsum, 2);
        float sc = dsum;
        if constexpr (Q) {
          const float s =
              (float)__builtin_bit_cast(_Float16, uint16_t(R.km[u] & 0xffffu)) * FI::scale_mul;
          sc = s * dsum;
          if constexpr (ZP) {
            const float z = (float)__builtin_bit_cast(_Float16, uint16_t(R.km[u] >> 16));
            sc = s * dsum + z * qsum[j];
          }
        }
        x[u][j] = sc * a.scale_log2;
        if (tail && !pm.valid(tr + 16 * u)) x[u][j] = -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mloc = x[0][j];
#pragma unroll
      for (int u = 1; u < TPL; ++u) mloc = fmaxf(mloc, x[u][j]);
      mloc = wave_max(mloc);
      const float mnew = fmaxf(m[j], mloc);
      const float al = fast_exp2(m[j] - mnew);
      m[j] = mnew;
      float ps = 0.0f, zs = 0.0f;
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        const float p = fast_exp2(x[u][j] - mnew);
        const bool valid = !tail || pm.valid(tr + 16 * u);
        float pv = p;
        if constexpr (Q) {
          const float vs =
              (float)__builtin_bit_cast(_Float16, uint16_t(R.vm[u] & 0xffffu)) * FI::scale_mul;
          pv = valid ? p * vs : 0.0f;
          if constexpr (ZP) {
            const float vz = (float)__builtin_bit_cast(_Float16, uint16_t(R.vm[u] >> 16));
            zs += valid ? p * vz : 0.0f;
          }
        }
        ps += p;
        if (c == 0) pbuf[j * P + tr + 16 * u] = pv;
      }
      lsum[j] = lsum[j] * al + (c == 0 ? ps : 0.0f);
      zacc[j] = zacc[j] * al + (c == 0 ? zs : 0.0f);
#pragma unroll
      for (int e = 0; e < DV; ++e) acc[j][e] *= al;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P.V: this lane's output channels d = lane*DV + e over all P tokens.
    float vv[DV][P];
    {
      uint32_t wv[VL * 4];
      __builtin_memcpy(wv, R.v, sizeof(R.v));
#pragma unroll
      for (int e = 0; e < DV; ++e)
#pragma unroll
        for (int t = 0; t < P; ++t) {
          float f;
          if constexpr (F == kBF16) {
            const int idx = e * P + t;
            f = bf16_to_f32((wv[idx >> 1] >> (16 * (idx & 1))) & 0xffffu);
            if (tail && !pm.valid(t)) f = 0.0f;
          } else if constexpr (F == kI4) {
            // byte t of the pair row; this channel's nibble
            const int nib = DV == 2 ? e : (lane & 1);
            f = code_to_f32<F>((wv[t >> 2] >> (8 * (t & 3))) >> (4 * nib));
          } else {
            const int idx = e * P + t;
            f = code_to_f32<F>(wv[idx >> 2] >> (8 * (idx & 3)));
          }
          vv[e][t] = f;
        }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int t4 = 0; t4 < P / 4; ++t4) {
        const float4 pp = *reinterpret_cast<const float4*>(pbuf + j * P + 4 * t4);
#pragma unroll
        for (int e = 0; e < DV; ++e) {
          acc[j][e] += pp.x * vv[e][4 * t4] + pp.y * vv[e][4 * t4 + 1] +
                       pp.z * vv[e][4 * t4 + 2] + pp.w * vv[e][4 * t4 + 3];
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };

  if (wr.cnt > 0) {
    Regs ring[DEPTH];
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) issue(ring[s], min(s, wr.cnt - 1));
    for (int k0 = 0; k0 < wr.cnt; k0 += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        const int k = k0 + s;
        if (k < wr.cnt) compute(ring[s], k);
        issue(ring[s], min(k + DEPTH, wr.cnt - 1));
      }
    }
  }

#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float lt = wave_sum_f(lsum[j]);
    const float zt = ZP ? wave_sum_f(zacc[j]) : 0.0f;
#pragma unroll
    for (int e = 0; e < DV; ++e) sm_o[(wave * G + j) * D + lane * DV + e] = acc[j][e] + zt;
    if (lane == 0) {
      sm_m[wave * G + j] = m[j];
      sm_l[wave * G + j] = lt;
    }
  }
  __syncthreads();
  combine_and_store<D, SCHED>(a, wr, sm_o, sm_m, sm_l, W, G);
}

template <int F, int P, int D, int G, int DEPTH, bool SCHED>
__global__ __launch_bounds__(valu_max_threads(P, D, G)) void decode_valu_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  if constexpr (!SCHED) {
    valu_item<F, P, D, G, DEPTH, false>(a, work_range<P>(a, wave, W), smem);
  } else {
    const int i0 = max(a.sched[8 + blockIdx.x], 0);
    const int i1 = min(a.sched[9 + blockIdx.x], a.num_items);
    for (int i = i0; i < i1; ++i) {
      if (!item_valid(a, i)) continue;
      valu_item<F, P, D, G, DEPTH, true>(a, item_range<P>(a, i, wave, W), smem);
      __syncthreads();  // the next item reuses the LDS merge and probability buffers
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of split partials, one wavefront per output row:
// M = max_s m_s; w_s = l_s 2^(m_s - M); out = sum_s w_s o_s / sum_s w_s.
// Partial s of the row: o at po + s*so (D floats), (m, l) at pml + s*sml;
// S >= 1.
template <int D, int kPre>
__device__ __forceinline__ void lse_merge_row_pre(const float* __restrict__ po, int64_t so,
                                                  const float* __restrict__ pml, int64_t sml,
                                                  int S, uint16_t* __restrict__ out_row) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  // The first kPre slots' partials are loaded before anything else: they do
  // not depend on the weights, so their loads, those of (m, l) and the
  // maximum's exchange all overlap and the row pays one memory latency.
  // (Slots past S reload slot S - 1; their weights are 0, and adding the
  // zero terms leaves L and o unchanged.)
  float pre[kPre][E];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int64_t si = min(i, S - 1);
#pragma unroll
    for (int e = 0; e < E; ++e) pre[i][e] = po[si * so + lane * E + e];
  }
  // (m, l) of slot `lane` (the first 64 slots), loaded together; M over all
  float m0 = -INFINITY, l0 = 0.0f;
  if (lane < S) {
    m0 = pml[lane * sml];
    l0 = pml[lane * sml + 1];
  }
  float M = m0;
  for (int s = lane + 64; s < S; s += 64) M = fmaxf(M, pml[s * sml]);
  M = wave_max(M);
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.0f;
  float L = 0.0f;
  if (M != -INFINITY) {
    // weight of slot `lane`; empty slots (l = 0, m = -inf) weigh 0
    const float w0 = l0 > 0.0f ? l0 * fast_exp2(m0 - M) : 0.0f;
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w0), i));
      L += wi;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += wi > 0.0f ? wi * pre[i][e] : 0.0f;
    }
    for (int s0 = 0; s0 < S; s0 += 64) {
      float ms = m0, ls = l0;
      if (s0 > 0) {
        const int s = s0 + lane;
        ms = s < S ? pml[s * sml] : -INFINITY;
        ls = s < S ? pml[s * sml + 1] : 0.0f;
      }
      // weight of slot s0 + lane; empty slots (l = 0, m = -inf) weigh 0
      const float w = ls > 0.0f ? ls * fast_exp2(ms - M) : 0.0f;
      const int n = min(64, S - s0);
      // the partials' loads do not depend on the weights, so consecutive
      // slots' loads are in flight together
#pragma unroll 4
      for (int i = s0 == 0 ? kPre : 0; i < n; ++i) {
        const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i));
        L += wi;
        const float* p = po + (s0 + i) * so + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float x = p[e];
          o[e] += wi > 0.0f ? wi * x : 0.0f;
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) out_row[lane * E + e] = f32_to_bf16_rne(L > 0.0f ? o[e] / L : 0.0f);
}
// Sixteen slots' partials loaded ahead, thirty-two for rows with more slots.
// Measured, the whole scheduled decode call (stream kernel + merge): 16
// sequences of 16k-32k INT4 tokens (about 24 slots per merged row) 107.4 us
// loading 4 slots ahead, 104.5 with 16, 101.4 with 32; a ragged Llama-3-8B
// bfloat16 layer (2-3 slots per row) 119.0, 118.4 and 119.8.
template <int D>
__device__ __forceinline__ void lse_merge_row(const float* __restrict__ po, int64_t so,
                                              const float* __restrict__ pml, int64_t sml, int S,
                                              uint16_t* __restrict__ out_row) {
  if (S > 16)
    lse_merge_row_pre<D, 32>(po, so, pml, sml, S, out_row);
  else
    lse_merge_row_pre<D, 16>(po, so, pml, sml, S, out_row);
}

// Uniform plan: row = b*H_q + j holds its S partials at (row*S + s).
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    uint16_t* __restrict__ out, int rows, int S) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  lse_merge_row<D>(part_o + int64_t(row) * S * D, D, part_ml + int64_t(row) * S * 2, 2, S,
                   out + int64_t(row) * D);
}

// Balanced schedule: merge entry e = (sequence, KV head, first slot, count);
// query head j of its group has partial (slot*g + j) for each of its slots.
template <int D>
__global__ __launch_bounds__(256) void merge_sched_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          const int32_t* __restrict__ entries,
                                                          uint16_t* __restrict__ out, int rows,
                                                          int g, int num_q_heads, int num_seqs,
                                                          int num_slots) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int e = row / g, j = row - e * g;
  const int32_t* m = entries + int64_t(e) * 4;
  const int b = m[0], h = m[1], first = m[2], cnt = m[3];
  // entries that name rows or slots outside this call are skipped
  if (unsigned(b) >= unsigned(num_seqs) || unsigned(h) >= unsigned(num_q_heads / g) ||
      first < 0 || cnt < 1 || int64_t(first) + cnt > num_slots)
    return;
  const int64_t p0 = int64_t(first) * g + j;
  lse_merge_row<D>(part_o + p0 * D, int64_t(g) * D, part_ml + p0 * 2, int64_t(g) * 2, cnt,
                   out + (int64_t(b) * num_q_heads + int64_t(h) * g + j) * D);
}

// ---------------------------------------------------------------------------
// Host side.
constexpr int kDepth = 2;
// Pages a matrix-core wavefront keeps in flight (one wavefront per SIMD, so
// the ring alone hides the memory latency behind the page computations):
// INT4 pages are half the bytes of INT8 ones, so it keeps twice as many.
// INT8 pages carry the most per-page arithmetic (codes, scales and zero
// points), and a third page in flight measured 10% faster for them (192 ->
// 172 us on 16 sequences of 16k-32k tokens), while FP8 measured 5% slower
// with three and bfloat16 within noise.
template <int F> constexpr int mfma_depth() { return F == kI4 ? 4 : F == kI8 ? 3 : kDepth; }
// Instances for larger groups hold NT head tiles of accumulators and q
// operands; for 32-token pages of 128 channels their rings shrink so that
// they fit the register file (at the depths above, four head tiles spilled
// 500-1,200 bytes per lane).
template <int F, int P, int D, int NT> constexpr int mfma_depth_nt() {
  return (P == 32 && D == 128 && NT == 4) ? 1
         : (P == 32 && D == 128 && NT == 2) ? (mfma_depth<F>() < 2 ? mfma_depth<F>() : 2)
                                              : mfma_depth<F>();
}
// The stream kernel's ring: the split kernel's with one wavefront per SIMD,
// one page with more.
template <int F, int P, int D, int NT> constexpr int stream_depth() {
  // (the stream kernel's item bookkeeping costs registers too: four head
  // tiles of 16-token pages also keep at most two pages, and quantized ones
  // with four head tiles, and bfloat16 ones of 16-token pages of 128
  // channels, one page (INT4 with 32-token pages of 64 channels: two), which
  // keeps them free of spills)
  constexpr bool q4 = NT == 4 && (F != kBF16 || (P == 16 && D == 128));
  constexpr int d0 = (P == 16 && D == 128 && NT == 4 && mfma_depth_nt<F, P, D, NT>() > 2)
                         ? 2 : mfma_depth_nt<F, P, D, NT>();
  constexpr int d1 = q4 ? (d0 < (F == kI4 ? 2 : 1) ? d0 : (F == kI4 ? 2 : 1)) : d0;
  return stream_waves_per_simd<F, NT>() == 1 ? d1 : 1;
}

int cu_count_current_device();

template <int F, int P, int D, bool SCHED>
hipError_t launch_decode_pd(const DecodeArgs& a, bool mfma, int g, dim3 grid, dim3 block,
                            size_t lds, hipStream_t s) {
  discard_stale_error();
  const int nt = g <= 16 ? 1 : g <= 32 ? 2 : 4;
  const int max_threads = mfma ? mfma_max_threads(P, D, nt) : valu_max_threads(P, D, g);
  if (int(block.x) > max_threads) return hipErrorInvalidConfiguration;
  if (mfma) {
    // balanced schedule: one stream per wavefront, no LDS
    if constexpr (SCHED) {
      if (g <= 16)
        hipLaunchKernelGGL((decode_mfma_stream_kernel<F, P, D, 1, stream_depth<F, P, D, 1>()>), grid, block,
                           0, s, a);
      else if (g <= 32)
        hipLaunchKernelGGL((decode_mfma_stream_kernel<F, P, D, 2, stream_depth<F, P, D, 2>()>), grid, block,
                           0, s, a);
      else
        hipLaunchKernelGGL((decode_mfma_stream_kernel<F, P, D, 4, stream_depth<F, P, D, 4>()>), grid, block,
                           0, s, a);
    } else {
      if (g <= 16)
        hipLaunchKernelGGL((decode_mfma_kernel<F, P, D, 1, mfma_depth_nt<F, P, D, 1>()>), grid, block, lds,
                           s, a);
      else if (g <= 32)
        hipLaunchKernelGGL((decode_mfma_kernel<F, P, D, 2, mfma_depth_nt<F, P, D, 2>()>), grid, block, lds,
                           s, a);
      else
        hipLaunchKernelGGL((decode_mfma_kernel<F, P, D, 4, mfma_depth_nt<F, P, D, 4>()>), grid, block, lds,
                           s, a);
    }
  } else {
    if (g == 1)
      hipLaunchKernelGGL((decode_valu_kernel<F, P, D, 1, kDepth, SCHED>), grid, block, lds, s,
                         a);
    else if (g == 2)
      hipLaunchKernelGGL((decode_valu_kernel<F, P, D, 2, kDepth, SCHED>), grid, block, lds, s,
                         a);
    else
      hipLaunchKernelGGL((decode_valu_kernel<F, P, D, 3, kDepth, SCHED>), grid, block, lds, s,
                         a);
  }
  return hipGetLastError();
}

// Instance for the pool's (page size, head dim); the descriptor was validated.
template <int F, bool SCHED>
hipError_t launch_decode_fmt(const DecodeArgs& a, int P, int D, bool mfma, int g, dim3 grid,
                             dim3 block, size_t lds, hipStream_t s) {
  if (P == 16)
    return D == 64 ? launch_decode_pd<F, 16, 64, SCHED>(a, mfma, g, grid, block, lds, s)
                   : launch_decode_pd<F, 16, 128, SCHED>(a, mfma, g, grid, block, lds, s);
  return D == 64 ? launch_decode_pd<F, 32, 64, SCHED>(a, mfma, g, grid, block, lds, s)
                 : launch_decode_pd<F, 32, 128, SCHED>(a, mfma, g, grid, block, lds, s);
}

}  // namespace kvp
