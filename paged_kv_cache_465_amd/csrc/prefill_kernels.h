// Multi-query paged attention (chunked prefill, verification of drafted
// tokens) for gfx950.
//
// A sequence holds n tokens in its pages; its last q_len are the new chunk,
// already written by kv_append.  Query row i of the chunk sits at position
// n - q_len + i and attends to positions 0 .. n - q_len + i ("KV-Cache
// Optimization Techniques", section "PagedAttention", eq. 1, restricted to
// the positions before and at the row; section "Cache-Aware Scheduling":
// long prompts are processed in chunks against the cache).  Query head j
// reads KV head j / g (section "Multi-Query and Grouped-Query Caching").
//
// Work decomposition.  For one (sequence, KV head) the rows are the pairs
// (chunk token i, head j of the group), row m = i * g + j.  A workgroup of
// four wavefronts owns a tile of 4 * 16 * NT consecutive rows; each wavefront
// owns 16 * NT of them and streams, with a register ring, every page up to
// the last position its rows see, 32 tokens per step (two 16-token pages, or
// one 32-token page).  The matrix-core tiles are the decode kernel's for
// 32-token pages: S^T = K q^T and O^T += V^T P^T on 16x16x32; a lane holds
// one row per tile, so the causal limit is a per-lane bound and the online
// softmax stays lane-local.  The wavefronts of
// a workgroup read the same pages at the same time, and all tiles of one
// (sequence, KV head) are placed on the same XCD, so page loads are ordinary
// (cacheable) loads that the tiles share through that XCD's L2.
//
// Short chunks (all rows of an item fit one wavefront, e.g. a few drafted
// tokens to verify): the four wavefronts each take all rows and a quarter of
// the pages instead, and wavefront 0 merges the four (m, l, o) partials
// through LDS, so no wavefront idles while one streams every page.
#pragma once
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "kvp.h"

namespace kvp {

struct PrefillArgs {
  const uint16_t* q;
  const int32_t* q_start;  // [B + 1]
  const void* k_pool;
  const void* v_pool;
  const uint16_t* k_meta;
  const uint16_t* v_meta;
  const int32_t* bt;
  const int32_t* ctx_lens;
  uint16_t* out;
  int32_t num_seqs, max_blocks, num_kv_heads, num_q_heads, group, num_pages, tiles;
  int32_t ctx_cap;
  float scale_log2;
  const int32_t* order;  // nullptr: natural grid order; else the unit of each workgroup
  int32_t units;         // workgroups of the natural grid
};

// Index, in the natural grid, of the unit this workgroup computes: its own
// position, or the entry a host-built schedule puts there.  Entries outside
// [0, units) are padding (nothing to do).
__device__ __forceinline__ int prefill_unit(const PrefillArgs& a) {
  return a.order ? a.order[blockIdx.x] : int(blockIdx.x);
}

// Tiled mode is bound by instruction issue.  Two workgroups per CU (two
// wavefronts per SIMD, <= 256 registers each) hide each other's dependency
// stalls; with a one-step ring (a step is 32 tokens: two 16-token pages) the
// budget holds without spills.  Measured on 512-token chunks of a
// Llama-3-8B-shaped layer (16-token pages): one workgroup per CU with
// 16-token steps 1216 us, two per CU 1005 us, paired steps at one per CU
// 944 us, paired steps with a one-step ring at two per CU 800 us.  Pages of
// 32 tokens x 128 channels do not fit two per CU; they keep one workgroup
// per CU and a two-step ring.
constexpr bool prefill_big_step(int P, int D) { return P == 32 && D == 128; }
constexpr int prefill_tiled_wg_per_cu(int P, int D) { return prefill_big_step(P, D) ? 1 : 2; }
constexpr int prefill_tiled_depth(int P, int D) { return prefill_big_step(P, D) ? 2 : 1; }

template <int BYTES> struct PrefillLoad;
template <> struct PrefillLoad<4> { using type = uint32_t; };
template <> struct PrefillLoad<8> { using type = uint2; };
template <> struct PrefillLoad<16> { using type = uint4; };

template <typename T>
__device__ __forceinline__ T load_plain(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

template <int F, int P, int D, int NT, int DEPTH, bool SPLIT>
__global__ __launch_bounds__(256, SPLIT ? 1 : prefill_tiled_wg_per_cu(P, D)) void
prefill_mfma_kernel(PrefillArgs a) {
  using FI = FmtInfo<F>;
  constexpr bool Q = FI::quant, ZP = FI::zero;
  // One step of the page loop covers VP tokens: one page, or in tiled mode
  // with 16-token pages two consecutive pages, so that P.V runs on the
  // 16x16x32 matrix-core shape (the 16x16x16 one does half the work per
  // instruction) and the softmax bookkeeping is paid once per 32 tokens.
  constexpr bool PAIR = P == 16 && !SPLIT;  // (split mode: measured no faster paired)
  constexpr int VP = PAIR ? 2 * P : P;
  constexpr int NSUB = VP / P;  // pages per step
  constexpr int T = VP / 16, KK = D / 32, NC = D / 16, EV = 4 * T;
  constexpr int RB = D * FI::bits / 8;   // bytes of one stored token row
  // K bytes a lane holds per 16-token sub-tile: bfloat16, KK pieces of 8
  // channels 32 apart (16 bytes each, 64 bytes apart); codes, D/4 contiguous
  // channels (D/4 bytes for 8-bit codes, D/8 for INT4)
  constexpr int KB = Q ? (D / 4) * FI::bits / 8 : 16 * KK;
  constexpr int KLB = KB >= 16 ? 16 : KB;   // bytes per K load
  constexpr int KN = KB / KLB;              // K loads per sub-tile
  constexpr int KSTEP = Q ? KLB : 64;       // byte distance between them
  // V^T bytes a lane holds per 16-channel chunk: EV tokens of one channel
  // (for INT4 the bytes of the channel pair holding it)
  constexpr int VB = F == kBF16 ? EV * 2 : EV;
  constexpr int ROWS_WAVE = 16 * NT;
  using OpA = typename std::conditional<Q, f16x8_t, bf16x8_t>::type;
  using OpPV = typename std::conditional<
      T == 1, typename std::conditional<Q, f16x4_t, bf16x4_t>::type, OpA>::type;
  using KLoad = typename PrefillLoad<KLB>::type;
  using VLoad = typename PrefillLoad<VB>::type;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, gq = lane >> 4;
  const int H = a.num_kv_heads, g = a.group;

  // Grid: groups of eight (sequence, KV head) items; within a group the index
  // runs tile-major, so workgroup i goes to XCD i mod 8 = item mod 8 and all
  // tiles of an item share one XCD (and its L2).  A schedule permutes the
  // units and keeps each item's tiles on one XCD.
  const int unit = prefill_unit(a);
  if (unit < 0 || unit >= a.units) return;   // the whole workgroup: no barrier reached
  const int per_group = 8 * a.tiles;
  const int grp = unit / per_group;
  const int within = unit - grp * per_group;
  const int tile = within >> 3;
  const int item = grp * 8 + (within & 7);
  if (item >= a.num_seqs * H) return;
  const int b = item / H, h = item - b * H;
  const int q0 = a.q_start[b];
  const int qlen = a.q_start[b + 1] - q0;
  const int ctx = min(max(a.ctx_lens[b], 0), a.ctx_cap);
  const int rows = qlen * g;
  const int row0 = SPLIT ? 0 : tile * 4 * ROWS_WAVE + wave * ROWS_WAVE;
  // whole wavefront (tiled) or workgroup (split: b is the workgroup's) idle;
  // the only barrier below is the split mode's, reached by all or none
  if (qlen <= 0 || row0 >= rows) return;
  const int row_last = min(row0 + ROWS_WAVE, rows) - 1;
  const int first_pos = ctx - qlen;       // position of chunk row 0
  // every row of this wavefront sees positions <= lim_min: steps ending there
  // (inside the sequence, all pages present) need no mask
  const int lim_min = first_pos + row0 / g;
  const int pos_last = min(first_pos + row_last / g, ctx - 1);
  const int nblk_all = pos_last >= 0 ? pos_last / VP + 1 : 0;    // steps
  const int npages = pos_last >= 0 ? pos_last / P + 1 : 0;        // pages they cover
  // blocks [kb0, kb0 + nblk) of this wavefront: all, or a quarter (split)
  const int cw = SPLIT ? (nblk_all + 3) / 4 : nblk_all;
  const int kb0 = SPLIT ? min(wave * cw, nblk_all) : 0;
  const int nblk = SPLIT ? max(0, min(cw, nblk_all - kb0)) : nblk_all;

  // This lane's row in each tile: its query (B operand of S^T = K q^T) and
  // its causal limit (positions <= lim take part).
  OpA qop[NT][KK];
  float qsum[NT];
  int lim[NT];
  bool live[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int m = row0 + nt * 16 + r;
    live[nt] = m < rows;
    const int mm = live[nt] ? m : row_last;
    const int i = mm / g, j = mm - (mm / g) * g;
    lim[nt] = first_pos + i;
    const uint16_t* qrow = a.q + ((int64_t(q0) + i) * a.num_q_heads + int64_t(h) * g + j) * D;
    float qs = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int d0 = Q ? (D / 4) * gq + 8 * kk : 32 * kk + 8 * gq;
      const uint4 raw = *reinterpret_cast<const uint4*>(qrow + d0);
      if constexpr (!Q) {
        qop[nt][kk] = __builtin_bit_cast(bf16x8_t, raw);
      } else {
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
        f16x8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = F == kI4 ? kI4KSlot(e) : e;  // the K operand's channel order
          const float f = bf16_to_f32((w4[c >> 1] >> (16 * (c & 1))) & 0xffffu);
          v[e] = (_Float16)f;
          qs += f;
        }
        qop[nt][kk] = v;
      }
    }
    qsum[nt] = ZP ? group4_sum(qs) : 0.0f;
  }

  // K rows: step token tok = page (tok / P) of the step, row tok % P.
  int koff[T], ksub[T];
#pragma unroll
  for (int st = 0; st < T; ++st) {
    const int tok = (T == 1) ? r : 8 * (r >> 2) + 4 * st + (r & 3);
    koff[st] = (tok % P) * RB + (Q ? KB * gq : 16 * gq);
    ksub[st] = tok / P;
  }
  // this lane's P.V (and score) tokens EV*gq .. EV*gq + EV - 1 lie in one
  // page of the step
  const int vsub = (EV * gq) / P;
  const int vcol = (EV * gq) % P;
  // V^T tile: [D][P] elements, or [D/2][P] bytes for INT4 (channel pairs)
  const int voff = F == kBF16 ? (r * P + vcol) * 2 : (F == kI4 ? (r >> 1) * P : r * P) + vcol;
  constexpr int vstride = F == kBF16 ? 16 * P * 2 : (F == kI4 ? 8 * P : 16 * P);
  const int moff = vcol * 4;
  const size_t tile_bytes = size_t(P) * RB;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int32_t* btrow = a.bt + int64_t(b) * a.max_blocks;

  struct Regs {
    KLoad k[T][KN];
    VLoad v[NC];
    uint4 km[Q ? T : 1];
    uint4 vm[Q ? T : 1];
    int phys[NSUB];  // -1: page absent (outside the pool, or past the rows' range)
  };
  auto issue = [&](Regs& R, int k) {
    int64_t tt[NSUB];
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      const int pg = k * NSUB + u;
      const int phys = pg < npages ? btrow[pg] : -1;
      const bool ok = unsigned(phys) < unsigned(a.num_pages);
      R.phys[u] = ok ? phys : -1;
      tt[u] = int64_t(ok ? phys : 0) * H + h;
    }
    // per lane: the page of the step its K rows / V tokens come from
    auto tile_of = [&](int sub) { return NSUB == 1 || sub == 0 ? tt[0] : tt[NSUB - 1]; };
    const int64_t t = tile_of(vsub);
    const char* vp = vbase + t * tile_bytes;
    const char* kps[T];
#pragma unroll
    for (int st = 0; st < T; ++st) kps[st] = kbase + tile_of(ksub[st]) * tile_bytes;
    // the per-token metadata first: the V scales decide the step's operand
    // offset before its scores, and waiting for them does not wait for codes
    if constexpr (Q) {
      const char* km = reinterpret_cast<const char*>(a.k_meta) + t * (P * 4);
      const char* vm = reinterpret_cast<const char*>(a.v_meta) + t * (P * 4);
#pragma unroll
      for (int st = 0; st < T; ++st) {
        R.vm[st] = *reinterpret_cast<const uint4*>(vm + moff + st * 16);
        R.km[st] = *reinterpret_cast<const uint4*>(km + moff + st * 16);
      }
    }
    // tiled: the workgroup's wavefronts share each page through L2 (ordinary
    // loads); split: each page is read once (non-temporal loads)
    if constexpr (!SPLIT) {
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < KN; ++i)
          R.k[st][i] = load_plain<KLoad>(kps[st] + koff[st] + i * KSTEP);
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) R.v[nc] = load_plain<VLoad>(vp + voff + nc * vstride);
    } else {
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < KN; ++i)
          R.k[st][i] = load_stream<KLoad>(kps[st] + koff[st] + i * KSTEP);
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) R.v[nc] = load_stream<VLoad>(vp + voff + nc * vstride);
    }
  };

  float m[NT], lsum[NT], zacc[NT];
  f32x4_t acc[NT][NC];
  // quantized pools: the largest V-scale exponent seen, which sets the
  // power-of-two offset 2^c the weights carry (vexp_offset); lsum, zacc and
  // acc are in units of 2^c
  int vexp = 0;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    lsum[nt] = 0.0f;
    zacc[nt] = 0.0f;
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) acc[nt][nc] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  auto compute = [&](const Regs& R, int k) {
    // absent pages: their tokens do not take part
    bool any_page = false;
#pragma unroll
    for (int u = 0; u < NSUB; ++u) any_page |= R.phys[u] >= 0;
    if (!any_page) return;
    // this lane's tokens' page (a select, not a register-array index)
    const bool page_ok = (NSUB > 1 && vsub) ? R.phys[NSUB - 1] >= 0 : R.phys[0] >= 0;
    bool all_pages = true;
#pragma unroll
    for (int u = 0; u < NSUB; ++u) all_pages &= R.phys[u] >= 0;
    const int base = k * VP;
    const int rem = ctx - base;  // rows of this page inside the sequence (>= 1)
    // wave-uniform: the whole step lies inside the sequence, below every
    // row's causal limit, on present pages
    const bool unmasked = all_pages && rem >= VP && base + VP - 1 <= lim_min;
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
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kop[st][kk] = codes8_to_f16x8<F>(w + DW * kk);
      }
    }
    OpPV vop[NC];
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) {
      if constexpr (!Q) {
        VLoad raw = R.v[nc];
        if (rem < VP || !page_ok) {
          // rows past the sequence may hold anything (NaN): zero them
          uint32_t wv[EV / 2];
          __builtin_memcpy(wv, &raw, sizeof(raw));
#pragma unroll
          for (int e = 0; e < EV; ++e)
            if (EV * gq + e >= rem || !page_ok) wv[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          __builtin_memcpy(&raw, wv, sizeof(raw));
        }
        vop[nc] = __builtin_bit_cast(OpPV, raw);
      } else {
        uint32_t wv[EV / 4];
        __builtin_memcpy(wv, &R.v[nc], sizeof(R.v[nc]));
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
    float ks[T][4], kz[T][4], vs[T][4], vz[T][4];
    if constexpr (Q) {
#pragma unroll
      for (int st = 0; st < T; ++st) {
        const uint32_t kw[4] = {R.km[st].x, R.km[st].y, R.km[st].z, R.km[st].w};
        const uint32_t vw[4] = {R.vm[st].x, R.vm[st].y, R.vm[st].z, R.vm[st].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ks[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(kw[i] & 0xffffu)) * FI::scale_mul;
          kz[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(kw[i] >> 16));
          vs[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(vw[i] & 0xffffu)) * FI::scale_mul;
          vz[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(vw[i] >> 16));
        }
      }
    }
    // the offset c, raised only when a V scale of this step's tokens (those
    // inside the sequence, on present pages) has a larger exponent than any
    // before (wave-uniform)
    int cnew = vexp_offset(vexp), cdelta = 0;
    if constexpr (Q) {
      float vmax = 0.0f;
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool valid = unmasked || (EV * gq + 4 * st + i < rem && page_ok);
          vmax = fmaxf(vmax, valid ? vs[st][i] : 0.0f);
        }
      if (wave_any(__float_as_uint(vmax) >= uint32_t(vexp + 1) << 23)) {
        vmax = group4_max(vmax);
        const int e = __builtin_amdgcn_readfirstlane(int(__float_as_uint(vmax) >> 23));
        const int cold = cnew;
        vexp = max(vexp, e);
        cnew = vexp_offset(vexp);
        cdelta = cnew - cold;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float x[T][4];
#pragma unroll
      for (int st = 0; st < T; ++st) {
        f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) sc = mfma_16x16x32(kop[st][kk], qop[nt][kk], sc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = ZP  ? (ks[st][i] * sc[i] + kz[st][i] * qsum[nt]) * a.scale_log2
                          : Q ? ks[st][i] * sc[i] * a.scale_log2
                              : sc[i] * a.scale_log2;
          x[st][i] = v;
        }
      }
      if (!unmasked) {
#pragma unroll
        for (int st = 0; st < T; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = base + EV * gq + 4 * st + i;
            // causal: this lane's row sees positions <= lim (and < ctx)
            if (!(tok <= lim[nt] && tok < ctx && page_ok)) x[st][i] = -INFINITY;
          }
      }
      float mloc = x[0][0];
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, x[st][i]);
      mloc = group4_max(mloc);
      const float mnew = fmaxf(m[nt], mloc);
      // a row none of whose positions has been seen yet keeps m = -inf: use 0
      // as the reference so that no (-inf) - (-inf) arises
      const float mref = mnew == -INFINITY ? 0.0f : mnew;
      const float al = fast_exp2(Q ? (m[nt] - mref) + float(cdelta) : m[nt] - mref);
      m[nt] = mnew;
      // weights 2^(score - m + c)
      const float mref_c = Q ? mref - float(cnew) : mref;
      float p[T][4];
      float ps = 0.0f;
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[st][i] = fast_exp2(x[st][i] - mref_c);
          ps += p[st][i];
        }
      lsum[nt] = lsum[nt] * al + ps;
      // once the running maximum settles, al is exactly 1 for every row:
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
            const int t = kV4Slot<F>(i);  // slot i holds token t, the V^T operand's order
            const bool valid = EV * gq + 4 * st + t < rem && page_ok;
            const float pv = valid ? p[st][t] * vs[st][t] : 0.0f;
            if constexpr (ZP) zs += valid ? p[st][t] * vz[st][t] : 0.0f;
            pop[4 * st + i] = (_Float16)pv;
          }
        if constexpr (ZP) zacc[nt] = zacc[nt] * al + zs;
      } else {
#pragma unroll
        for (int st = 0; st < T; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) pop[4 * st + i] = (__bf16)p[st][i];
      }
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) {
        if constexpr (T == 1)
          acc[nt][nc] = mfma_16x16x16(vop[nc], pop, acc[nt][nc]);
        else
          acc[nt][nc] = mfma_16x16x32(vop[nc], pop, acc[nt][nc]);
      }
    }
  };

  if (nblk > 0) {
    Regs ring[DEPTH];
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) issue(ring[s], kb0 + min(s, nblk - 1));
    for (int k0 = 0; k0 < nblk; k0 += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        const int k = k0 + s;
        if (k < nblk) compute(ring[s], kb0 + k);
        issue(ring[s], kb0 + min(k + DEPTH, nblk - 1));
      }
    }
  }

  if constexpr (SPLIT) {
    // waves 1..3 leave (o, m, l) of their pages in LDS, in the matrix-core
    // register layout; wave 0 merges them into its own and writes the rows
    __shared__ f32x4_t sm_o[3][NT][NC][64];
    __shared__ float sm_m[3][NT][64], sm_l[3][NT][64];
    // each wavefront's sums in plain units (their offsets 2^c differ)
    const float unc = exp2_int(-vexp_offset(vexp));
    if (wave > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float lt = group4_sum(lsum[nt]) * unc;
        const float zt = ZP ? group4_sum(zacc[nt]) : 0.0f;
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) {
          f32x4_t v = acc[nt][nc];
          if constexpr (ZP) v += zt;
          sm_o[wave - 1][nt][nc][lane] = v * unc;
        }
        sm_m[wave - 1][nt][lane] = m[nt];
        sm_l[wave - 1][nt][lane] = lt;
      }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float l0 = group4_sum(lsum[nt]) * unc;
      const float z0 = ZP ? group4_sum(zacc[nt]) : 0.0f;
      float M = m[nt];
#pragma unroll
      for (int w = 0; w < 3; ++w) M = fmaxf(M, sm_m[w][nt][lane]);
      // weights of the four partials (0 for one that saw no position)
      float f[4];
      f[0] = m[nt] == -INFINITY ? 0.0f : fast_exp2(m[nt] - M);
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const float mw = sm_m[w][nt][lane];
        f[w + 1] = mw == -INFINITY ? 0.0f : fast_exp2(mw - M);
      }
      float L = l0 * f[0];
#pragma unroll
      for (int w = 0; w < 3; ++w) L += sm_l[w][nt][lane] * f[w + 1];
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) {
        f32x4_t v = acc[nt][nc];
        if constexpr (ZP) v += z0;
        v *= f[0] * unc;
#pragma unroll
        for (int w = 0; w < 3; ++w) v += sm_o[w][nt][nc][lane] * f[w + 1];
        acc[nt][nc] = v;
      }
      lsum[nt] = L;  // merged row sum (already over the four lane groups)
    }
  }

  // Finalize: each lane's row is its own; out = acc / l (bfloat16, RNE).
  // (Split mode: acc and lsum already hold the merged sums, zero terms in.)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = SPLIT ? lsum[nt] : group4_sum(lsum[nt]);
    const float zt = (ZP && !SPLIT) ? group4_sum(zacc[nt]) : 0.0f;
    const int mrow = row0 + nt * 16 + r;
    if (mrow < rows) {
      const int i = mrow / g, j = mrow - (mrow / g) * g;
      uint16_t* orow =
          a.out + ((int64_t(q0) + i) * a.num_q_heads + int64_t(h) * g + j) * D;
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) {
        f32x4_t v = acc[nt][nc];
        if constexpr (ZP) v += zt;
        uint32_t lo = uint32_t(f32_to_bf16_rne(lt > 0.0f ? v[0] * inv : 0.0f)) |
                      (uint32_t(f32_to_bf16_rne(lt > 0.0f ? v[1] * inv : 0.0f)) << 16);
        uint32_t hi = uint32_t(f32_to_bf16_rne(lt > 0.0f ? v[2] * inv : 0.0f)) |
                      (uint32_t(f32_to_bf16_rne(lt > 0.0f ? v[3] * inv : 0.0f)) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * nc + 4 * gq) = make_uint2(lo, hi);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Row-tiled mode, K/V shared through LDS.
//
// A workgroup of WAVES wavefronts owns 32 RT WAVES consecutive rows of one
// (sequence, KV head); each wavefront owns RT tiles of 32 rows.  The key axis is walked in blocks of 64
// keys (four 16-token pages or two 32-token pages): all 256 threads load a
// block's K rows and V^T rows once into LDS (double-buffered: the next
// block's loads are in flight while the current one is computed) and every
// wavefront reads its matrix-core operands from there, so each page is read
// once per workgroup instead of once per wavefront.  This mode serves
// bfloat16 pools.  (Quantized pools keep the register-streaming tiled kernel
// above: rounding their dequantized K rows to a 16-bit operand moved scores
// by up to 1e-3 in log units at the workloads' x8 outlier channels, enough
// to push outputs past 1e-2; that kernel applies the per-token scales in
// float32 to exact codes.)
//
// Tiles are 32x32x16 matrix-core steps: S^T (64 keys x 32 rows) = K Q^T in two
// 32-key tiles, then O^T (D x 32 rows) += V^T P^T in four 16-key steps.  A
// lane owns one row (column n = lane % 32 of every accumulator), so the
// online softmax is lane-local but for one exchange with lane n + 32, which
// holds the row's other keys.  The score tile's row r of tile t is fed by key
// 32t + 16(j/2) + 8h + 4(j%2) + i (r = 8j + 4h + i), so that a lane's
// accumulator holds, for P.V step s, the 8 consecutive keys 16s + 8h .. + 7
// that its P^T operand needs: the V^T operand is then one 16-byte LDS read.
// Rows of LDS are padded by 16 bytes so the wavefront's reads of 32 different
// rows at one column spread over the banks.
template <int D, int WAVES>
struct FaTile {
  static constexpr int NT = 64 * WAVES;           // threads of a workgroup
  static constexpr int KEYS = 64;                 // keys per block
  static constexpr int W = D / 8;                 // 16-byte chunks of one K row (8 values)
  static constexpr int KROW = (W + 1) * 16;       // LDS bytes per K row (padded)
  static constexpr int VROW = (KEYS / 8 + 1) * 16;  // LDS bytes per V^T row (padded)
  static constexpr int KBLK = KEYS * KROW;
  static constexpr int STAGE = KBLK + D * VROW;   // one block of K and V^T
  static constexpr int KCH = KEYS * W / NT;       // K chunks each thread stages per block
  static constexpr int VCH = D * (KEYS / 8) / NT;  // V^T chunks each thread stages
  static constexpr int KS = D / 16;               // 32x32x16 steps over the head dim
  static constexpr int DT = D / 32;               // 32-channel output tiles
};

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ f32x16_t mfma_32x32x16(const bf16x8_t& a, const bf16x8_t& b,
                                                  const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max(x, x of lane n ^ 32): lanes n and n + 32 hold two halves of one row.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int P, int D, int WAVES, int RT>
__global__ __launch_bounds__(64 * WAVES, (WAVES == 4 && RT == 1) ? 2 : 1) void prefill_fa_kernel(
    PrefillArgs a) {
  using TL = FaTile<D, WAVES>;
  constexpr int NT = TL::NT;
  constexpr int KEYS = TL::KEYS, W = TL::W, KS = TL::KS, DT = TL::DT;
  constexpr int RB = D * 2;                       // bytes of one stored token row
  constexpr int PPB = KEYS / P;                   // pages per block
  using Op = bf16x8_t;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * TL::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int H = a.num_kv_heads, g = a.group;

  // Grid as the tiled kernel: all tiles of an item on one XCD.
  const int unit = prefill_unit(a);
  if (unit < 0 || unit >= a.units) return;   // the whole workgroup: no barrier reached
  const int per_group = 8 * a.tiles;
  const int grp = unit / per_group;
  const int within = unit - grp * per_group;
  const int tile = within >> 3;
  const int item = grp * 8 + (within & 7);
  if (item >= a.num_seqs * H) return;
  const int b = item / H, h = item - b * H;
  const int q0 = a.q_start[b];
  const int qlen = a.q_start[b + 1] - q0;
  const int ctx = min(max(a.ctx_lens[b], 0), a.ctx_cap);
  const int rows = qlen * g;
  constexpr int WROWS = 32 * RT;                  // rows of one wavefront
  const int wg_row0 = tile * WROWS * WAVES;
  if (qlen <= 0 || wg_row0 >= rows) return;       // the whole workgroup: no barrier reached
  const int first_pos = ctx - qlen;
  const int wg_row_last = min(wg_row0 + WROWS * WAVES - 1, rows - 1);
  const int wg_pos_last = min(first_pos + wg_row_last / g, ctx - 1);
  const int nblk = wg_pos_last >= 0 ? wg_pos_last / KEYS + 1 : 0;

  // this wavefront's rows: tile rt holds rows row0 + 32 rt .. + 31
  const int row0 = wg_row0 + wave * WROWS;
  const bool wave_live = row0 < rows;
  const int row_last = wave_live ? min(row0 + WROWS - 1, rows - 1) : wg_row_last;
  const int wpos_min = first_pos + (wave_live ? row0 : wg_row_last) / g;
  const int wpos_max = first_pos + row_last / g;
  int m_row[RT], qi[RT], qj[RT], lim[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_row[rt] = row0 + 32 * rt + n;
    const int mm = m_row[rt] < rows ? m_row[rt] : row_last;  // rows past the end mirror the last
    qi[rt] = mm / g;
    qj[rt] = mm - qi[rt] * g;
    lim[rt] = first_pos + qi[rt];                            // keys <= lim take part (< ctx)
  }

  // Q^T as the B operand of S^T = K Q^T: lane (n, hh) holds channels 16ks + 8hh .. + 7.
  // A negative scale is applied as |scale| on -q (exact), so that the running
  // maximum of the raw scores is the maximum of the scaled ones.
  const float cs = fabsf(a.scale_log2);
  const uint32_t qflip = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
  Op qop[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const uint16_t* qrow =
        a.q + ((int64_t(q0) + qi[rt]) * a.num_q_heads + int64_t(h) * g + qj[rt]) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hh);
      raw.x ^= qflip;
      raw.y ^= qflip;
      raw.z ^= qflip;
      raw.w ^= qflip;
      qop[rt][ks] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  // LDS read bases: K row of score-tile row r = n for tile t; V^T row d = n of tile dt.
  int kread[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = n >> 3, ih = (n >> 2) & 1, i = n & 3;
    const int key = 32 * t + 16 * (j >> 1) + 8 * ih + 4 * (j & 1) + i;
    kread[t] = key * TL::KROW + hh * 16;
  }
  const int vread = TL::KBLK + n * TL::VROW + hh * 16;
  // key offsets (within a block) of this lane's score values, tile t, value r
  auto key_of = [&](int t, int r) {
    return 32 * t + 16 * (r >> 3) + 8 * hh + 4 * ((r >> 2) & 1) + (r & 3);
  };

  // ---- staging: this thread's K chunks (key, column chunk) and V^T chunks
  // (channel, 8-key group); the column / key group is the same for all of them
  const int kcc = tid % W;
  const int vkc = tid & 7;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int32_t* btrow = a.bt + int64_t(b) * a.max_blocks;
  const size_t tile_bytes = size_t(P) * RB;
  const int npages_seq = (ctx + P - 1) / P;
  uint4 kraw[TL::KCH], vraw[TL::VCH];
  int vphys;
  // Page ids of a block's PPB pages, loaded one block ahead of its staging
  // (raw table words, uniform in-range index) so that no load waits on a
  // table entry; validated (-1: absent, past the sequence or past the last
  // block) when the block is staged.
  struct PageTab { int raw[PPB]; int blk; };
  auto load_tab = [&](int blk) {
    PageTab t;
    t.blk = blk;
#pragma unroll
    for (int pi = 0; pi < PPB; ++pi) {
      const int lb = __builtin_amdgcn_readfirstlane(min(blk * PPB + pi, npages_seq - 1));
      t.raw[pi] = btrow[max(lb, 0)];
    }
    return t;
  };
  // (a vector, not an array: a lane-dependent pick among the ids is then an
  // in-register selection, never a stack slot)
  typedef int PageVec __attribute__((ext_vector_type(PPB)));
  struct PageIds { PageVec id; bool clean; };  // clean: every page present, every key < ctx
  auto validate = [&](const PageTab& t) {
    PageIds v;
    v.clean = t.blk < nblk && (t.blk + 1) * KEYS <= ctx;
#pragma unroll
    for (int pi = 0; pi < PPB; ++pi) {
      const int lb = t.blk * PPB + pi;
      const bool ok = t.blk < nblk && lb < npages_seq && unsigned(t.raw[pi]) < unsigned(a.num_pages);
      v.id[pi] = __builtin_amdgcn_readfirstlane(ok ? t.raw[pi] : -1);
      v.clean = v.clean && ok;
    }
    return v;
  };
  // block-local page of this thread's K chunk c (the same for every lane when
  // a chunk round covers at most one page)
  auto kpage = [&](int c) {
    constexpr int KPR = NT / W;    // keys per chunk round
    return KPR <= P ? (c * KPR) / P : (c * KPR + tid / W) / P;
  };
  auto sel = [](const PageIds& v, int pi) {
    return v.id[pi];
  };
  auto stage_load = [&](const PageIds& ids) {
#pragma unroll
    for (int c = 0; c < TL::KCH; ++c) {
      const int key = (c * NT + tid) / W;
      const int phys = sel(ids, kpage(c));
      const int64_t t = int64_t(phys < 0 ? 0 : phys) * H + h;
      kraw[c] = *reinterpret_cast<const uint4*>(kbase + t * tile_bytes + (key % P) * RB + kcc * 16);
    }
    const int phys = sel(ids, (8 * vkc) / P);
    vphys = phys;
    const int64_t t = int64_t(phys < 0 ? 0 : phys) * H + h;
    const int tok0 = (8 * vkc) % P;
#pragma unroll
    for (int c = 0; c < TL::VCH; ++c) {
      const int d = (c * NT + tid) >> 3;
      vraw[c] = *reinterpret_cast<const uint4*>(vbase + t * tile_bytes + (d * P + tok0) * 2);
    }
  };
  auto stage_store = [&](int blk, const PageIds& ids, unsigned char* st) {
    if (ids.clean) {   // wave-uniform: no key of the block needs zeroing
#pragma unroll
      for (int c = 0; c < TL::KCH; ++c)
        *reinterpret_cast<uint4*>(st + ((c * NT + tid) / W) * TL::KROW + kcc * 16) = kraw[c];
#pragma unroll
      for (int c = 0; c < TL::VCH; ++c)
        *reinterpret_cast<uint4*>(st + TL::KBLK + ((c * NT + tid) >> 3) * TL::VROW + vkc * 16) =
            vraw[c];
      return;
    }
    const int key0 = blk * KEYS;
#pragma unroll
    for (int c = 0; c < TL::KCH; ++c) {
      const int key = (c * NT + tid) / W;
      const bool ok = sel(ids, kpage(c)) >= 0 && key0 + key < ctx;
      *reinterpret_cast<uint4*>(st + key * TL::KROW + kcc * 16) =
          ok ? kraw[c] : make_uint4(0, 0, 0, 0);
    }
    // V^T: keys 8 vkc .. + 7 of channel d; keys past the sequence (or on an
    // absent page) are zero so that their zero weights never meet NaN
    const int kv0 = key0 + 8 * vkc;
#pragma unroll
    for (int c = 0; c < TL::VCH; ++c) {
      const int d = (c * NT + tid) >> 3;
      uint32_t w[4];
      __builtin_memcpy(w, &vraw[c], 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool keep = vphys >= 0 && kv0 + e < ctx;
        w[e >> 1] &= keep ? 0xffffffffu : ((e & 1) ? 0x0000ffffu : 0xffff0000u);
      }
      uint4 v;
      __builtin_memcpy(&v, w, 16);
      *reinterpret_cast<uint4*>(st + TL::KBLK + d * TL::VROW + vkc * 16) = v;
    }
  };

  // ---- online softmax state (this lane's rows, its half of each block's keys)
  float m[RT], lsum[RT];
  f32x16_t acc[RT][DT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    lsum[rt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = f32x16_t{};
  }

  auto compute = [&](int blk, const PageIds& ids, const unsigned char* st) {
    const int key0 = blk * KEYS;
    if (!wave_live || key0 > wpos_max) return;   // wave-uniform: nothing of this block is seen
    // pages of the block present? (wave-uniform)
    uint32_t pmask = 0;
#pragma unroll
    for (int pi = 0; pi < PPB; ++pi) pmask |= (ids.id[pi] >= 0 ? 1u : 0u) << pi;
    const bool unmasked = pmask == (1u << PPB) - 1 && key0 + KEYS - 1 <= wpos_min;
    // All score tiles' matrix-core steps are issued first (each K operand read
    // from LDS feeds the RT row tiles); the softmax of one tile then runs on
    // the vector ALU while later tiles' steps execute.  Each 32-key tile is
    // one step of the online softmax; its P.V steps read each V^T operand
    // once for the RT row tiles.
    f32x16_t sc[RT][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sc[rt][t] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const Op kop = *reinterpret_cast<const Op*>(st + kread[t] + 32 * ks);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sc[rt][t] = mfma_32x32x16(kop, qop[rt][ks], sc[rt][t]);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      Op pop[RT][2];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x16_t& x = sc[rt][t];
        if (!unmasked) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = key_of(t, r);
            const bool ok = key0 + kk <= lim[rt] && ((pmask >> (kk / P)) & 1u);
            x[r] = ok ? x[r] : -INFINITY;
          }
        }
        float mx = x[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
        mx = pair_max(mx) * cs;
        // The softmax reference m only moves when a score exceeds it by more
        // than 2^8 (log2 units): weights stay <= 256 (exact enough in
        // bfloat16, no float32 overflow in the sums) and the accumulators are
        // rescaled rarely.
        const float mnew = mx > m[rt] + 8.0f ? mx : m[rt];
        // a row that has seen no key yet keeps m = -inf: use 0 as the reference
        const float mref = mnew == -INFINITY ? 0.0f : mnew;
        const float al = fast_exp2(m[rt] - mref);
        m[rt] = mnew;
        float ps = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(x[r] * cs - mref);
          x[r] = p;
          ps += p;
        }
        lsum[rt] = lsum[rt] * al + ps;
        if (wave_any(al != 1.0f)) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= al;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int e = 0; e < 8; ++e) pop[rt][half][e] = (__bf16)x[8 * half + e];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int step = 2 * t + half;   // keys 16 step .. + 15
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const Op vop =
              *reinterpret_cast<const Op*>(st + vread + dt * 32 * TL::VROW + 32 * step);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt][dt] = mfma_32x32x16(vop, pop[rt][half], acc[rt][dt]);
        }
      }
    }
  };

  if (nblk > 0) {
    PageIds ids_cur = validate(load_tab(0));
    PageTab tab_next = load_tab(1);
    stage_load(ids_cur);
    stage_store(0, ids_cur, lds);
    __syncthreads();
    for (int blk = 0; blk < nblk; ++blk) {
      unsigned char* cur = lds + (blk & 1) * TL::STAGE;
      unsigned char* nxt = lds + ((blk + 1) & 1) * TL::STAGE;
      const bool more = blk + 1 < nblk;
      const PageIds ids_next = validate(tab_next);
      if (more) stage_load(ids_next);
      compute(blk, ids_cur, cur);
      // (issued after the compute: its wait would otherwise share the LDS
      // reads' counter at the first matrix-core step)
      tab_next = load_tab(blk + 2);
      if (more) stage_store(blk + 1, ids_next, nxt);
      __syncthreads();
      ids_cur = ids_next;
    }
  }

  // ---- finalize: out = acc / l, bfloat16
  if (!wave_live) return;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lt = pair_sum(lsum[rt]);
    if (m_row[rt] >= rows) continue;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    uint16_t* orow =
        a.out + ((int64_t(q0) + qi[rt]) * a.num_q_heads + int64_t(h) * g + qj[rt]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16_t& v = acc[rt][dt];
        const uint32_t lo = uint32_t(f32_to_bf16_rne(v[4 * j + 0] * inv)) |
                            (uint32_t(f32_to_bf16_rne(v[4 * j + 1] * inv)) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16_rne(v[4 * j + 2] * inv)) |
                            (uint32_t(f32_to_bf16_rne(v[4 * j + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * j + 4 * hh) = make_uint2(lo, hi);
      }
  }
}

constexpr int kPrefillDepth = 2;  // split mode
// wavefronts per workgroup of the LDS-staged kernel (32 rows each): four,
// two workgroups per compute unit (eight, one per compute unit, measured
// 25% slower on 512-token chunks)
constexpr int kFaWaves = 4;
// 32-row tiles per wavefront: one.  (Two, with one wavefront per SIMD for
// the registers, measured 38% slower on 512-token chunks: a lone wavefront
// does not overlap its softmax with its matrix-core steps.)
constexpr int kFaRowTiles = 1;

template <int F, int P, int D>
hipError_t launch_prefill_pd(const PrefillArgs& a, int nt, bool split, dim3 grid, hipStream_t s) {
  discard_stale_error();
  if (split) {
    if (nt == 1)
      hipLaunchKernelGGL((prefill_mfma_kernel<F, P, D, 1, kPrefillDepth, true>), grid,
                         dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_mfma_kernel<F, P, D, 2, kPrefillDepth, true>), grid,
                         dim3(256), 0, s, a);
  } else if constexpr (F == kBF16) {
    hipLaunchKernelGGL((prefill_fa_kernel<P, D, kFaWaves, kFaRowTiles>), grid, dim3(64 * kFaWaves),
                       0, s, a);
  } else {
    if (nt == 1)
      hipLaunchKernelGGL((prefill_mfma_kernel<F, P, D, 1, prefill_tiled_depth(P, D), false>), grid,
                         dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_mfma_kernel<F, P, D, 2, prefill_tiled_depth(P, D), false>), grid,
                         dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// Instance for the pool's (page size, head dim); the descriptor was validated.
template <int F>
hipError_t launch_prefill_fmt(const PrefillArgs& a, int P, int D, int nt, bool split, dim3 grid,
                              hipStream_t s) {
  if (P == 16)
    return D == 64 ? launch_prefill_pd<F, 16, 64>(a, nt, split, grid, s)
                   : launch_prefill_pd<F, 16, 128>(a, nt, split, grid, s);
  return D == 64 ? launch_prefill_pd<F, 32, 64>(a, nt, split, grid, s)
                 : launch_prefill_pd<F, 32, 128>(a, nt, split, grid, s);
}

}  // namespace kvp
