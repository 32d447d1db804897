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

template <bool INT8, int P, int D, int NT, int DEPTH, bool SPLIT>
__global__ __launch_bounds__(256, SPLIT ? 1 : prefill_tiled_wg_per_cu(P, D)) void
prefill_mfma_kernel(PrefillArgs a) {
  // One step of the page loop covers VP tokens: one page, or in tiled mode
  // with 16-token pages two consecutive pages, so that P.V runs on the
  // 16x16x32 matrix-core shape (the 16x16x16 one does half the work per
  // instruction) and the softmax bookkeeping is paid once per 32 tokens.
  constexpr bool PAIR = P == 16 && !SPLIT;  // (split mode: measured no faster paired)
  constexpr int VP = PAIR ? 2 * P : P;
  constexpr int NSUB = VP / P;  // pages per step
  constexpr int T = VP / 16, KK = D / 32, NC = D / 16, EV = 4 * T;
  constexpr int EB = INT8 ? 1 : 2;
  constexpr int KL = INT8 ? D / 64 : KK;
  constexpr int VB = EV * EB;
  constexpr int ROWS_WAVE = 16 * NT;
  using OpA = typename std::conditional<INT8, f16x8_t, bf16x8_t>::type;
  using OpPV = typename std::conditional<
      T == 1, typename std::conditional<INT8, f16x4_t, bf16x4_t>::type, OpA>::type;
  using VLoad = typename std::conditional<VB == 4, uint32_t,
                typename std::conditional<VB == 8, uint2, uint4>::type>::type;

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
      const int d0 = INT8 ? (D / 4) * gq + 8 * kk : 32 * kk + 8 * gq;
      const uint4 raw = *reinterpret_cast<const uint4*>(qrow + d0);
      if constexpr (!INT8) {
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
    qsum[nt] = INT8 ? group4_sum(qs) : 0.0f;
  }

  // K rows: step token tok = page (tok / P) of the step, row tok % P.
  int koff[T], ksub[T];
#pragma unroll
  for (int st = 0; st < T; ++st) {
    const int tok = (T == 1) ? r : 8 * (r >> 2) + 4 * st + (r & 3);
    koff[st] = ((tok % P) * D + (INT8 ? (D / 4) * gq : 8 * gq)) * EB;
    ksub[st] = tok / P;
  }
  // this lane's P.V (and score) tokens EV*gq .. EV*gq + EV - 1 lie in one
  // page of the step
  const int vsub = (EV * gq) / P;
  const int vcol = (EV * gq) % P;
  const int voff = (r * P + vcol) * EB;
  const int moff = vcol * 4;
  const size_t tile_bytes = size_t(P) * D * EB;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int32_t* btrow = a.bt + int64_t(b) * a.max_blocks;

  struct Regs {
    uint4 k[T][KL];
    VLoad v[NC];
    uint4 km[INT8 ? T : 1];
    uint4 vm[INT8 ? T : 1];
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
        for (int i = 0; i < KL; ++i)
          R.k[st][i] = *reinterpret_cast<const uint4*>(kps[st] + koff[st] + i * (INT8 ? 16 : 64));
#pragma unroll
      for (int nc = 0; nc < NC; ++nc)
        R.v[nc] = *reinterpret_cast<const VLoad*>(vp + voff + nc * 16 * P * EB);
    } else {
#pragma unroll
      for (int st = 0; st < T; ++st)
#pragma unroll
        for (int i = 0; i < KL; ++i)
          R.k[st][i] = load_stream<uint4>(kps[st] + koff[st] + i * (INT8 ? 16 : 64));
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) R.v[nc] = load_stream<VLoad>(vp + voff + nc * 16 * P * EB);
    }
    if constexpr (INT8) {
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
      if constexpr (!INT8) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kop[st][kk] = __builtin_bit_cast(bf16x8_t, R.k[st][kk]);
      } else {
#pragma unroll
        for (int i = 0; i < KL; ++i) {
          const uint32_t w4[4] = {R.k[st][i].x, R.k[st][i].y, R.k[st][i].z, R.k[st][i].w};
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            f16x2_t a0, a1, b0, b1;
            i8x4_to_f16x4(w4[2 * half], a0, a1);
            i8x4_to_f16x4(w4[2 * half + 1], b0, b1);
            kop[st][2 * i + half] = f16x8_t{a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
          }
        }
      }
    }
    OpPV vop[NC];
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) {
      if constexpr (!INT8) {
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
          i8x4_to_f16x4(wv[i], lo, hi);
          v[4 * i + 0] = lo[0];
          v[4 * i + 1] = lo[1];
          v[4 * i + 2] = hi[0];
          v[4 * i + 3] = hi[1];
        }
        vop[nc] = v;
      }
    }
    float ks[T][4], kz[T][4], vs[T][4], vz[T][4];
    if constexpr (INT8) {
#pragma unroll
      for (int st = 0; st < T; ++st) {
        const uint32_t kw[4] = {R.km[st].x, R.km[st].y, R.km[st].z, R.km[st].w};
        const uint32_t vw[4] = {R.vm[st].x, R.vm[st].y, R.vm[st].z, R.vm[st].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ks[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(kw[i] & 0xffffu));
          kz[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(kw[i] >> 16));
          vs[st][i] = (float)__builtin_bit_cast(_Float16, uint16_t(vw[i] & 0xffffu));
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
          const float v = INT8 ? (ks[st][i] * sc[i] + kz[st][i] * qsum[nt]) * a.scale_log2
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
      if constexpr (INT8) {
        float zs = 0.0f;
#pragma unroll
        for (int st = 0; st < T; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool valid = EV * gq + 4 * st + i < rem && page_ok;
            const float pv = valid ? p[st][i] * vs[st][i] : 0.0f;
            zs += valid ? p[st][i] * vz[st][i] : 0.0f;
            pop[4 * st + i] = (_Float16)pv;
          }
        zacc[nt] = zacc[nt] * al + zs;
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
        const float zt = INT8 ? group4_sum(zacc[nt]) : 0.0f;
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) {
          f32x4_t v = acc[nt][nc];
          if constexpr (INT8) v += zt;
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
      const float z0 = INT8 ? group4_sum(zacc[nt]) : 0.0f;
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
        if constexpr (INT8) v += z0;
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
    const float zt = (INT8 && !SPLIT) ? group4_sum(zacc[nt]) : 0.0f;
    const int mrow = row0 + nt * 16 + r;
    if (mrow < rows) {
      const int i = mrow / g, j = mrow - (mrow / g) * g;
      uint16_t* orow =
          a.out + ((int64_t(q0) + i) * a.num_q_heads + int64_t(h) * g + j) * D;
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
      for (int nc = 0; nc < NC; ++nc) {
        f32x4_t v = acc[nt][nc];
        if constexpr (INT8) v += zt;
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

template <bool INT8, int P, int D>
hipError_t launch_prefill_pd(const PrefillArgs& a, int nt, bool split, dim3 grid, hipStream_t s) {
  discard_stale_error();
  if (split) {
    if (nt == 1)
      hipLaunchKernelGGL((prefill_mfma_kernel<INT8, P, D, 1, kPrefillDepth, true>), grid,
                         dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_mfma_kernel<INT8, P, D, 2, kPrefillDepth, true>), grid,
                         dim3(256), 0, s, a);
  } else {
    if (nt == 1)
      hipLaunchKernelGGL((prefill_mfma_kernel<INT8, P, D, 1, prefill_tiled_depth(P, D), false>), grid,
                         dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_mfma_kernel<INT8, P, D, 2, prefill_tiled_depth(P, D), false>), grid,
                         dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvp

extern "C" kvp_status kvp_paged_attention_prefill(
    const kvp_pool* pool, const void* q, const int32_t* q_start, const void* k_pool,
    const void* v_pool, const void* k_meta, const void* v_meta, const int32_t* block_tables,
    int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_q_len, int32_t max_context_len, float scale, void* out, kvp_stream_t stream) {
  using namespace kvp;
  kvp_pool_desc d;
  if (kvp_pool_get_desc(pool, &d) != KVP_OK) return KVP_E_INVAL;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks <= 0 || max_q_len < 0) return KVP_E_INVAL;
  if (num_q_heads % d.num_kv_heads) return KVP_E_INVAL;
  if (int64_t(max_blocks) * d.page_size > 0x7fffffff) return KVP_E_INVAL;
  if (max_context_len < 0 || int64_t(max_context_len) > int64_t(max_blocks) * d.page_size)
    return KVP_E_INVAL;
  if (!std::isfinite(scale)) return KVP_E_INVAL;
  const int g = num_q_heads / d.num_kv_heads;
  if (g > 64) return KVP_E_UNSUPPORTED;
  if (num_seqs == 0 || max_q_len == 0) return KVP_OK;
  if (!q || !q_start || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return KVP_E_INVAL;
  // the multi-query kernel reads bfloat16 and INT8 pools
  if (d.dtype != KVP_BF16 && d.dtype != KVP_INT8) return KVP_E_UNSUPPORTED;
  const bool int8 = d.dtype == KVP_INT8;
  if (int8 != (k_meta != nullptr) || int8 != (v_meta != nullptr)) return KVP_E_INVAL;
  // rows per wavefront: 32 when the longest chunk has at least that many rows;
  // chunks whose rows fit one wavefront split the pages across the four
  const int64_t max_rows = int64_t(max_q_len) * g;
  const bool split = max_rows <= 32;
  const int nt = split ? (max_rows > 16 ? 2 : 1) : (max_rows >= 32 * 4 ? 2 : 1);
  const int64_t rows_wg = split ? 16 * nt : 4 * 16 * nt;
  const int64_t tiles = (max_rows + rows_wg - 1) / rows_wg;
  const int64_t items = int64_t(num_seqs) * d.num_kv_heads;
  const int64_t wgs = (items + 7) / 8 * 8 * tiles;
  if (tiles > 0x7fffffff || wgs > 0x7fffffff) return KVP_E_UNSUPPORTED;
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_start = q_start;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_meta = static_cast<const uint16_t*>(k_meta);
  a.v_meta = static_cast<const uint16_t*>(v_meta);
  a.bt = block_tables;
  a.ctx_lens = context_lens;
  a.out = static_cast<uint16_t*>(out);
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks;
  a.num_kv_heads = d.num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.group = g;
  a.num_pages = d.num_pages;
  a.tiles = int32_t(tiles);
  a.ctx_cap = max_context_len;
  a.scale_log2 = scale * kLog2e;
  const dim3 grid(static_cast<unsigned>(wgs));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  const int key = (d.page_size == 32) * 4 + (d.head_dim == 128) * 2 + int8;
  switch (key) {
    case 0: e = launch_prefill_pd<false, 16, 64>(a, nt, split, grid, s); break;
    case 1: e = launch_prefill_pd<true, 16, 64>(a, nt, split, grid, s); break;
    case 2: e = launch_prefill_pd<false, 16, 128>(a, nt, split, grid, s); break;
    case 3: e = launch_prefill_pd<true, 16, 128>(a, nt, split, grid, s); break;
    case 4: e = launch_prefill_pd<false, 32, 64>(a, nt, split, grid, s); break;
    case 5: e = launch_prefill_pd<true, 32, 64>(a, nt, split, grid, s); break;
    case 6: e = launch_prefill_pd<false, 32, 128>(a, nt, split, grid, s); break;
    default: e = launch_prefill_pd<true, 32, 128>(a, nt, split, grid, s); break;
  }
  return e == hipSuccess ? KVP_OK : KVP_E_HIP;
}
