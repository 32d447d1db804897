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
};

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
  // tiles of an item share one XCD (and its L2).
  const int per_group = 8 * a.tiles;
  const int grp = blockIdx.x / per_group;
  const int within = blockIdx.x - grp * per_group;
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
          const float f = bf16_to_f32((w4[e >> 1] >> (16 * (e & 1))) & 0xffffu);
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
    if constexpr (Q) {
      const char* km = reinterpret_cast<const char*>(a.k_meta) + t * (P * 4);
      const char* vm = reinterpret_cast<const char*>(a.v_meta) + t * (P * 4);
#pragma unroll
      for (int st = 0; st < T; ++st) {
        R.km[st] = *reinterpret_cast<const uint4*>(km + moff + st * 16);
        R.vm[st] = *reinterpret_cast<const uint4*>(vm + moff + st * 16);
      }
    }
  };

  float m[NT], lsum[NT], zacc[NT];
  f32x4_t acc[NT][NC];
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
      const float al = fast_exp2(m[nt] - mref);
      m[nt] = mnew;
      float p[T][4];
      float ps = 0.0f;
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[st][i] = fast_exp2(x[st][i] - mref);
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
            const bool valid = EV * gq + 4 * st + i < rem && page_ok;
            const float pv = valid ? p[st][i] * vs[st][i] : 0.0f;
            if constexpr (ZP) zs += valid ? p[st][i] * vz[st][i] : 0.0f;
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
    if (wave > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float lt = group4_sum(lsum[nt]);
        const float zt = ZP ? group4_sum(zacc[nt]) : 0.0f;
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) {
          f32x4_t v = acc[nt][nc];
          if constexpr (ZP) v += zt;
          sm_o[wave - 1][nt][nc][lane] = v;
        }
        sm_m[wave - 1][nt][lane] = m[nt];
        sm_l[wave - 1][nt][lane] = lt;
      }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float l0 = group4_sum(lsum[nt]);
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
        v *= f[0];
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

constexpr int kPrefillDepth = 2;  // split mode

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
