// attend.hip — attention over the selected tokens only (split-K decoding).
//
// TokenSelect README, "Key Takeaways": only the selected critical tokens take
// part in the attention computation. For each query head h the softmax of
// scale*q_h.K[j] is renormalised over the selected rows j and applied to
// V[j]; one selection is shared by every head of the sequence.
//
// attend_kernel: one work-group per (split of the index list, KV head,
// sequence), with an online softmax in fp32, base 2, and (max, sum, acc[d])
// left per (sequence, head, split).
//  * bf16 rows (index lists and dense ranges): the GS query heads of a KV
//    head share every row, so the scores of a 64-token chunk are one small
//    matrix product (16 tokens x 16 padded heads per wave on
//    v_mfma_f32_16x16x32_bf16); the weights and V rows go through LDS and the
//    weighted sum is taken on the vector units, each (head, dimension pair)
//    owned by one thread.
//  * fp32 rows: a row group of LPR lanes gathers one token's K and V rows
//    (16-byte loads), takes the GS dot products and combines them with DPP;
//    row groups are merged through LDS in a fixed order.
// combine_kernel merges the splits by their log-sum-exp and, in a decode
// step, also updates the Selection-Cache state.
#include "topk_device.h"

namespace ts {

template <int DT, int D, int GS, bool PAGED, bool DENSE, bool SEL>
__global__ __launch_bounds__(256) void attend_kernel(AttendParams p) {
  constexpr int ESZ = DT ? 2 : 4;
  constexpr int ROWB = D * ESZ;
  constexpr int LPR = (ROWB / 16 < 16) ? ROWB / 16 : 16;  // lanes per row
  constexpr int CPL = ROWB / (16 * LPR);                   // 16-byte chunks per lane
  constexpr int EPC = 16 / ESZ;                            // elements per chunk
  constexpr int EPL = EPC * CPL;                           // elements per lane
  constexpr int W = 4 * CPL;                               // 32-bit words per lane
  constexpr int UA = 4;                                    // rows in flight per row group
  constexpr int RG = 256 / LPR;
  // bf16 rows take the matrix-core path below; fp32 rows the row-group path
  constexpr bool MF = DT == 1;
  // LDS rows of the matrix-core path: V rows of D/2 + 2 words (8-byte aligned;
  // rows 8 apart fall 16 banks apart, so the column reads of P * V do not
  // conflict), and bf16 weight parts in rows of 64 tokens per head (+4 words)
  constexpr int kVRow = D / 2 + 2;
  constexpr int kPtRow = 36;

  __shared__ float s_m[4][MF ? 1 : GS];
  __shared__ float s_l[4][MF ? 1 : GS];
  __shared__ float s_acc[MF ? 1 : 4 * GS * D];
  __shared__ __align__(16) uint32_t s_v[MF ? 64 * kVRow : 1];
  __shared__ __align__(16) uint32_t s_pt[MF ? 2 * 16 * kPtRow : 1];   // hi rows, then lo rows
  __shared__ float s_wm[MF ? 64 : 1];
  __shared__ float s_wl[MF ? 64 : 1];
  // decode steps: the end of the top-k for this split's token range
  __shared__ uint32_t s_ck[SEL ? kCandLds : 1];
  __shared__ uint32_t s_ci[SEL ? kCandLds : 1];
  __shared__ __align__(16) uint32_t s_hist[SEL ? 2048 : 1];
  __shared__ uint32_t s_rw[SEL ? kSelRangeMax / 32 : 1];
  __shared__ int32_t s_tok[SEL ? kSelRangeMax : (DENSE ? 1 : kAttendStage)];
  __shared__ uint32_t s_sh[16];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y / p.nslices;
  const int slice = blockIdx.y - kvh * p.nslices;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int j = tid % LPR;
  const int rg = tid / LPR;
  const int wv = tid >> 6, lane = tid & 63;
  const int len = p.seq_lens ? p.seq_lens[b] : p.len_base + b;
  const int bkv = p.kv_shared ? 0 : b;
  int pbeg = split * p.split;
  int pend = min(pbeg + p.split, p.nidx);
  const int32_t* idx =
      DENSE ? nullptr : p.idx + (size_t)b * p.idx_b_stride + (size_t)kvh * p.idx_kv_stride;
  const int Hkv = p.Hkv;
  // requested first, whatever the path (bf16 rows): the query fragments and
  // this lane's first list entry, so that on a hit step (or any list read
  // straight from global memory) neither waits behind the hit flag
  const int tl = lane & 15, g4 = lane >> 4;
  uint4 qf[MF ? D / 32 : 1];
  int raw0 = -1;
  if constexpr (MF) {
    const int head = kvh * p.G + slice * GS + min(tl, GS - 1);
    const char* qb = (const char*)p.q + ((size_t)b * p.Hq + head) * ROWB + g4 * 16;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const uint4 v = ld16(qb + s * 64);
      qf[s] = tl < GS ? v : make_uint4(0u, 0u, 0u, 0u);
    }
    if constexpr (!DENSE) {
      // (on a decode miss step the list is the stored selection that this
      // kernel is rewriting: the entry is then stale and not used)
      const int pos = pbeg + 16 * wv + tl;
      if (pos < pend) raw0 = idx[p.sel_page_log2 > 0 ? (pos >> p.sel_page_log2) : pos];
    }
  }
  bool lds_list = false;
  if constexpr (SEL) {
    if (!p.sel_hit[b]) {
      // ---- the selection of tokens [r0, r1): the partition kernel set the
      // bits of every key above the k-th key's histogram bin b0 (or of the
      // whole bin), listed the keys inside b0 and counted them by key bits
      // 19..10; the threshold inside b0 is found again here (every
      // work-group of the sequence gets the same one)
      const int k = p.sel_k;
      const int k_eff = min(k, len);
      const int r0 = split * p.sel_range;
      const int r1 = max(r0, min(r0 + p.sel_range, len));
      const uint32_t* ctrl = p.sel_ctrl + (size_t)b * kCtrlStride;
      const uint32_t* bm = p.sel_bitmap + (size_t)b * p.sel_bm_stride;
      const uint2* cand = p.sel_cand + (size_t)b * kCandCap;
      const uint32_t b0 = ctrl[kCtlPrefix], need = ctrl[kCtlNeed], C = ctrl[kCtlCandCount];
      uint2 cv[kCandLds / 256];
#pragma unroll
      for (int i = 0; i < kCandLds / 256; ++i) cv[i] = cand[i * 256 + tid];  // stale past C: unused
      // the partition kernel's histogram of key bits 19..10 over bin b0
      const uint4 hb = ld16(ctrl + kCtlHistB + 4 * tid);
      const int w0 = r0 >> 5, wr = (r1 - r0 + 31) >> 5;
      uint32_t rw = tid < wr ? bm[w0 + tid] : 0u;
      // selected base bits before the range: 16-byte loads of whole groups of
      // four words below w0 (the row's bitmap is 16-byte aligned), then single
      // words for a partial last group, so no word at or past w0 is counted
      uint32_t pc = 0;
      for (int w = 4 * tid; w < w0; w += 4 * 256) {
        if (w + 4 <= w0) {
          const uint4 q4 = *reinterpret_cast<const uint4*>(bm + w);
          pc += (__popc(q4.x) + __popc(q4.y)) + (__popc(q4.z) + __popc(q4.w));
        } else {
          for (int i = w; i < w0; ++i) pc += __popc(bm[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < kCandLds / 256; ++i) {
        s_ck[i * 256 + tid] = cv[i].x;
        s_ci[i * 256 + tid] = cv[i].y;
      }
      if (tid < wr) s_rw[tid] = rw;
      *reinterpret_cast<uint4*>(s_hist + 4 * tid) = hb;
      __syncthreads();
      if (need > 0 && k_eff > 0) {
        const float* vrow = p.sel_votes + (size_t)b * p.sel_vote_stride;
        auto visit = [&](const auto& L) {
          const BinThreshold th = find_threshold<256, true>(L, b0, need, s_hist, s_sh);
          for (int i = tid; i < L.size(); i += 256) {
            const uint2 e = L.get(i);
            if (th.take(e)) {
              if (e.y < (uint32_t)r0) ++pc;
              else if (e.y < (uint32_t)r1) atomicOr(&s_rw[(e.y >> 5) - w0], 1u << (e.y & 31));
            }
          }
        };
        if (C <= (uint32_t)kCandLds) visit(LdsList{s_ck, s_ci, (int)C});
        else if (C <= (uint32_t)kCandCap) visit(GlobalList{cand, (int)C});
        else visit(RowList{vrow, len});
      }
      __syncthreads();
      uint32_t before, count;
      (void)block_excl_scan<256>(pc, s_sh, &before);
      const uint32_t wbits = tid < wr ? s_rw[tid] : 0u;
      uint32_t o = block_excl_scan<256>(__popc(wbits), s_sh, &count);
      for (uint32_t m = wbits; m; m &= m - 1) s_tok[o++] = (w0 + tid) * 32 + (__ffs(m) - 1);
      __syncthreads();
      // this range's part of the ascending selection (one work-group per range)
      if (kvh == 0 && slice == 0) {
        int32_t* so = p.sel_out + (size_t)b * k;
        for (uint32_t i = tid; i < count; i += 256) so[before + i] = s_tok[i];
        if (split == 0)
          for (int i = max(k_eff, 0) + tid; i < k; i += 256) so[i] = -1;
      }
      lds_list = true;
      pbeg = 0;
      pend = (int)count;
    }
  }

  auto row_of = [&](int t) -> size_t {
    if constexpr (PAGED) {
      const int pg = p.page_table[(size_t)b * p.pt_stride + (t >> p.ps_log2)];
      return ((((size_t)pg << p.ps_log2) + (t & ((1 << p.ps_log2) - 1))) * Hkv + kvh);
    } else {
      return (((size_t)bkv * p.max_len + t) * Hkv + kvh);
    }
  };
  // UA rows (tokens tok[u]; -1 = none) into registers
  auto load_rows = [&](const int (&tok)[UA], uint32_t (&kw)[UA][W], uint32_t (&vw)[UA][W]) {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      {
        // tok is clamped into the sequence by every caller; validity is
        // tracked apart, so the loads are unconditional
        const size_t row = row_of(tok[u]);
        const char* kp = (const char*)p.k + row * ROWB;
        const char* vp = (const char*)p.v + row * ROWB;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const uint4 a = ld16(kp + (c * LPR + j) * 16);
          const uint4 v = ld16(vp + (c * LPR + j) * 16);
          kw[u][4 * c + 0] = a.x; kw[u][4 * c + 1] = a.y; kw[u][4 * c + 2] = a.z; kw[u][4 * c + 3] = a.w;
          vw[u][4 * c + 0] = v.x; vw[u][4 * c + 1] = v.y; vw[u][4 * c + 2] = v.z; vw[u][4 * c + 3] = v.w;
        }
      }
    }
  };

  // the row-group path (fp32 rows): GS query rows, running max, sum and acc
  uint32_t qw[GS][W];
  float m[GS], l[GS], acc[GS][EPL];
  // scores of a batch, one rescale of the running sums per batch
  auto consume = [&](const bool (&ok)[UA], const uint32_t (&kw)[UA][W], const uint32_t (&vw)[UA][W]) {
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      float sc[UA];
      float bm = m[hh];
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) a = fmaf(__uint_as_float(kw[u][w]), __uint_as_float(qw[hh][w]), a);
        sc[u] = ok[u] ? group_sum<LPR>(a) * p.scale2 : -INFINITY;
        bm = fmaxf(bm, sc[u]);
      }
      if (bm == -INFINITY) continue;           // nothing valid yet for this row group
      const float corr = ex2(m[hh] - bm);      // 0 when m was -inf
      float pw[UA];
      float ls = l[hh] * corr;
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        pw[u] = ex2(sc[u] - bm);               // 0 for invalid rows
        ls += pw[u];
      }
      l[hh] = ls;
      m[hh] = bm;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float a = acc[hh][e] * corr;
#pragma unroll
        for (int u = 0; u < UA; ++u) a = fmaf(pw[u], __uint_as_float(vw[u][e]), a);
        acc[hh][e] = a;
      }
    }
  };

  // token at list position pos of a global list (-1: none, or outside the
  // sequence), from the list entry `raw` that holds it
  auto tok_from = [&](int pos, int raw) -> int {
    if (pos >= pend) return -1;
    long long t;
    if (p.sel_page_log2 > 0)
      t = raw < 0 ? -1 : ((long long)raw << p.sel_page_log2) + (pos & ((1 << p.sel_page_log2) - 1));
    else
      t = raw;
    return (t >= 0 && t < len) ? (int)t : -1;
  };
  auto tok_at = [&](int pos) -> int {
    if (pos >= pend) return -1;
    return tok_from(pos, idx[p.sel_page_log2 > 0 ? (pos >> p.sel_page_log2) : pos]);
  };
  if constexpr (MF) {
    // ---- bf16 rows. Each wave takes 16 tokens of a 64-token chunk (lane l:
    // token l%16, dimensions 32s + 8*(l/16) .. +7 of its K and V rows, one
    // 16-byte load per k-step). The matrix cores give S^T = K_tile * Q^T for
    // the slice's heads padded to 16 (lane l: tokens 4*(l/16) .. +3, head
    // l%16). The chunk's max per head, the weights P = 2^(s - M) and the V
    // rows go through LDS, and the matrix cores add P * V_chunk into O (lane
    // l: heads 4*(l/16) .. +3, dimension l%16 of each of the wave's
    // 16-dimension tiles); V's columns are read from LDS 16 bits at a time.
    // P enters as two bf16 parts, hi = bf16(P) and lo = bf16(P - hi), so the
    // weights keep about 16 significant bits (fp32-level accuracy of the
    // output; V rows are bf16 already), and the row sums add the same hi + lo.
    constexpr int KS = D / 32;                 // k-steps of 32 dimensions
    constexpr int NTW = D / 64;                // 16-dimension tiles of O per wave
    float Mc = -INFINITY;                      // running max of head tl (score side)
    float Mo[4], Lo[4];                        // running max and sum of heads 4*g4 + i
    f32x4_t O[NTW];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Mo[i] = -INFINITY;
      Lo[i] = 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) O[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (len > 0) {
      constexpr int CAP = SEL ? kSelRangeMax : kAttendStage;
      // dense: the contiguous tokens [pbeg, min(pend, len)), no list
      const int n = DENSE ? max(0, min(pend, len) - pbeg) : pend - pbeg;
      const bool direct = DENSE || (!lds_list && n <= 64);
      for (int c0 = 0; c0 < n; c0 += CAP) {
        const int cn = min(CAP, n - c0);
        if (!lds_list && !direct) {
          __syncthreads();                     // the previous chunk's readers are done
          for (int i = tid; i < cn; i += 256) s_tok[i] = tok_at(pbeg + c0 + i);
          __syncthreads();
        }
        const int nit = (cn + 63) / 64;
        // this lane's row of chunk it (an empty slot reads token 0, masked)
        auto tok = [&](int it, bool& ok) -> int {
          const int q = it * 64 + 16 * wv + tl;
          int tt;
          if constexpr (DENSE) tt = pbeg + c0 + q;
          else if (direct && c0 == 0 && it == 0) tt = tok_from(pbeg + q, raw0);  // requested at the start
          else tt = direct ? tok_at(pbeg + c0 + q) : s_tok[min(q, cn - 1)];
          ok = q < cn && tt >= 0 && tt < len;
          return ok ? tt : 0;
        };
        auto load = [&](int t, uint4 (&kf)[KS], uint4 (&vf)[KS]) {
          const size_t row = row_of(t);
          const char* kp = (const char*)p.k + row * ROWB + g4 * 16;
          const char* vp = (const char*)p.v + row * ROWB + g4 * 16;
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            kf[s] = ld16(kp + s * 64);
            vf[s] = ld16(vp + s * 64);
          }
        };
        auto chunk = [&](int it, bool ok, const uint4 (&kf)[KS], const uint4 (&vf)[KS]) {
          f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) sc = mfma16(as_bf8(kf[s]), as_bf8(qf[s]), sc);
          const uint64_t okm = __ballot(ok);   // bit t < 16: token t of the wave is valid
          float sv[4], mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool v = (okm >> (4 * g4 + i)) & 1u;
            sv[i] = v ? sc[i] * p.scale2 : -INFINITY;
            mx = fmaxf(mx, sv[i]);
          }
          mx = xor_max<32>(xor_max<16>(mx));
          // V rows at LDS row 16*wv + tl (8-byte stores: the padded row is 8-byte aligned)
          uint32_t* vr = s_v + (16 * wv + tl) * kVRow + g4 * 4;
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            *reinterpret_cast<uint2*>(vr + s * 16) = make_uint2(vf[s].x, vf[s].y);
            *reinterpret_cast<uint2*>(vr + s * 16 + 2) = make_uint2(vf[s].z, vf[s].w);
          }
          if (g4 == 0) s_wm[wv * 16 + tl] = mx;
          __syncthreads();
          // weights of head tl as bf16 hi + lo parts, and their sum over the wave's tokens
          Mc = fmaxf(Mc, fmaxf(fmaxf(s_wm[tl], s_wm[16 + tl]), fmaxf(s_wm[32 + tl], s_wm[48 + tl])));
          uint32_t ph[4], pl[4];
          float ls = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pw = sv[i] == -INFINITY ? 0.f : ex2(sv[i] - Mc);
            ph[i] = bf16_bits(pw);
            const float hv = __uint_as_float(ph[i] << 16);
            pl[i] = bf16_bits(pw - hv);          // exact difference
            ls += hv + __uint_as_float(pl[i] << 16);
          }
          ls = xor_sum<32>(xor_sum<16>(ls));
          *reinterpret_cast<uint2*>(s_pt + tl * kPtRow + 8 * wv + 2 * g4) =
              make_uint2(ph[0] | (ph[1] << 16), ph[2] | (ph[3] << 16));
          *reinterpret_cast<uint2*>(s_pt + (16 + tl) * kPtRow + 8 * wv + 2 * g4) =
              make_uint2(pl[0] | (pl[1] << 16), pl[2] | (pl[3] << 16));
          if (g4 == 0) s_wl[wv * 16 + tl] = ls;
          // rescale this lane's rows of O (heads 4*g4 + i) to the new max
          float corr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = 4 * g4 + i;
            const float mn = fmaxf(Mo[i], fmaxf(fmaxf(s_wm[h], s_wm[16 + h]), fmaxf(s_wm[32 + h], s_wm[48 + h])));
            corr[i] = mn == -INFINITY ? 1.f : ex2(Mo[i] - mn);
            Mo[i] = mn;
          }
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[nt][i] *= corr[i];
          __syncthreads();
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = 4 * g4 + i;
            Lo[i] = Lo[i] * corr[i] + ((s_wl[h] + s_wl[16 + h]) + (s_wl[32 + h] + s_wl[48 + h]));
          }
          // O += P * V over the chunk's 64 tokens, two k-steps of 32
          const uint16_t* vh = reinterpret_cast<const uint16_t*>(s_v);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const uint4 pa = *reinterpret_cast<const uint4*>(s_pt + tl * kPtRow + 16 * ks + 4 * g4);
            const uint4 pb = *reinterpret_cast<const uint4*>(s_pt + (16 + tl) * kPtRow + 16 * ks + 4 * g4);
            const int r0 = 32 * ks + 8 * g4;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
              const int dim = 16 * (NTW * wv + nt) + tl;
              uint32_t w[4];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                w[j] = (uint32_t)vh[(r0 + 2 * j) * (2 * kVRow) + dim] |
                       ((uint32_t)vh[(r0 + 2 * j + 1) * (2 * kVRow) + dim] << 16);
              const bf16x8_t vb = as_bf8(make_uint4(w[0], w[1], w[2], w[3]));
              O[nt] = mfma16(as_bf8(pa), vb, O[nt]);
              O[nt] = mfma16(as_bf8(pb), vb, O[nt]);
            }
          }
          // the next chunk's V rows and weights overwrite these
          if (it + 1 < nit || c0 + CAP < n) __syncthreads();
        };
        uint4 kA[KS], vA[KS], kB[KS], vB[KS];
        bool okA, okB;
        load(tok(0, okA), kA, vA);
        int it = 0;
        for (; it + 2 < nit; it += 2) {
          load(tok(it + 1, okB), kB, vB);
          __builtin_amdgcn_sched_barrier(0);
          chunk(it, okA, kA, vA);
          __builtin_amdgcn_sched_barrier(0);
          load(tok(it + 2, okA), kA, vA);
          __builtin_amdgcn_sched_barrier(0);
          chunk(it + 1, okB, kB, vB);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (it + 1 < nit) {
          load(tok(it + 1, okB), kB, vB);
          chunk(it, okA, kA, vA);
          chunk(it + 1, okB, kB, vB);
        } else {
          chunk(it, okA, kA, vA);
        }
      }
    }
    // this lane's rows of O: heads 4*g4 + i, dimension tl of the wave's tiles
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g4 + i;
      if (h < GS) {
        const int head = kvh * p.G + slice * GS + h;
        const size_t o = ((size_t)b * p.Hq + head) * p.nsplit + split;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) p.pacc[o * D + 16 * (NTW * wv + nt) + tl] = O[nt][i];
        if (wv == 0 && tl == 0) {
          p.pm[o] = Mo[i];
          p.pl[o] = Lo[i];
        }
      }
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      const int head = kvh * p.G + slice * GS + hh;
      const char* qb = (const char*)p.q + ((size_t)b * p.Hq + head) * ROWB;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const uint4 v = ld16(qb + (c * LPR + j) * 16);
        qw[hh][4 * c + 0] = v.x; qw[hh][4 * c + 1] = v.y;
        qw[hh][4 * c + 2] = v.z; qw[hh][4 * c + 3] = v.w;
      }
    }
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
    }

    if constexpr (DENSE) {
      // contiguous token range [pbeg, pe): batches of RG*UA rows, the next
      // batch in flight while one is consumed; rows past the end are clamped
      // to the last token (in bounds) and masked, so every load is
      // unconditional and the compiler can count them
      const int pe = min(pend, len);
      const int nb = pe > pbeg ? (pe - pbeg + RG * UA - 1) / (RG * UA) : 0;
      uint32_t kA[UA][W], vA[UA][W], kB[UA][W], vB[UA][W];
      auto batch = [&](int bi, int (&t)[UA], bool (&ok)[UA]) {
#pragma unroll
        for (int u = 0; u < UA; ++u) {
          const int pos = pbeg + bi * RG * UA + u * RG + rg;
          ok[u] = pos < pe;
          t[u] = min(pos, pe - 1);
        }
      };
      int tA[UA], tB[UA];
      bool oA[UA], oB[UA];
      if (nb > 0) {
        batch(0, tA, oA);
        load_rows(tA, kA, vA);
      }
      int bi = 0;
      for (; bi + 2 < nb; bi += 2) {
        batch(bi + 1, tB, oB);
        load_rows(tB, kB, vB);
        __builtin_amdgcn_sched_barrier(0);
        consume(oA, kA, vA);
        __builtin_amdgcn_sched_barrier(0);
        batch(bi + 2, tA, oA);
        load_rows(tA, kA, vA);
        __builtin_amdgcn_sched_barrier(0);
        consume(oB, kB, vB);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (bi + 1 < nb) {
        batch(bi + 1, tB, oB);
        load_rows(tB, kB, vB);
        consume(oA, kA, vA);
        consume(oB, kB, vB);
      } else if (bi < nb) {
        consume(oA, kA, vA);
      }
    } else if (len > 0) {
      // The list's tokens go to LDS first (one round of index loads per chunk
      // of CAP positions; a decode step's own selection is there already);
      // then the rows stream through a two-stage pipeline whose loads are
      // unconditional: an empty slot reads token 0 and is masked.
      constexpr int CAP = SEL ? kSelRangeMax : kAttendStage;
      const int n = pend - pbeg;
      uint32_t kA[UA][W], vA[UA][W], kB[UA][W], vB[UA][W];
      int tA[UA], tB[UA];
      bool oA[UA], oB[UA];
      // a list of one batch is read straight from global memory (staging it
      // would only add a barrier)
      const bool direct = !lds_list && n <= RG * UA;
      for (int c0 = 0; c0 < n; c0 += CAP) {
        const int cn = min(CAP, n - c0);
        if (!lds_list && !direct) {
          __syncthreads();                         // the previous chunk's readers are done
          for (int i = tid; i < cn; i += 256) s_tok[i] = tok_at(pbeg + c0 + i);
          __syncthreads();
        }
        const int nit = (cn + RG * UA - 1) / (RG * UA);
        auto toks = [&](int it, int (&t)[UA], bool (&ok)[UA]) {
#pragma unroll
          for (int u = 0; u < UA; ++u) {
            const int q = it * RG * UA + u * RG + rg;
            const int tt = direct ? tok_at(pbeg + c0 + q) : s_tok[min(q, cn - 1)];
            ok[u] = q < cn && tt >= 0 && tt < len;
            t[u] = ok[u] ? tt : 0;
          }
        };
        toks(0, tA, oA);
        load_rows(tA, kA, vA);
        int it = 0;
        for (; it + 2 < nit; it += 2) {
          toks(it + 1, tB, oB);
          load_rows(tB, kB, vB);
          __builtin_amdgcn_sched_barrier(0);
          consume(oA, kA, vA);
          __builtin_amdgcn_sched_barrier(0);
          toks(it + 2, tA, oA);
          load_rows(tA, kA, vA);
          __builtin_amdgcn_sched_barrier(0);
          consume(oB, kB, vB);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (it + 1 < nit) {
          toks(it + 1, tB, oB);
          load_rows(tB, kB, vB);
          consume(oA, kA, vA);
          consume(oB, kB, vB);
        } else {
          consume(oA, kA, vA);
        }
      }
    }

    // merge the row groups (fixed order: deterministic): the common max and the
    // sums over a wave's row groups by lane swaps, over the 4 waves in LDS
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      float mw = m[hh];
      if constexpr (LPR <= 8) mw = xor_max<8>(mw);
      mw = xor_max<32>(xor_max<16>(mw));
      if (lane == 0) s_m[wv][hh] = mw;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      const float M = fmaxf(fmaxf(s_m[0][hh], s_m[1][hh]), fmaxf(s_m[2][hh], s_m[3][hh]));
      const float f = (l[hh] > 0.f) ? ex2(m[hh] - M) : 0.f;
      float lw = l[hh] * f;
      if constexpr (LPR <= 8) lw = xor_sum<8>(lw);
      lw = xor_sum<32>(xor_sum<16>(lw));
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float v = acc[hh][e] * f;
        if constexpr (LPR <= 8) v = xor_sum<8>(v);
        acc[hh][e] = xor_sum<32>(xor_sum<16>(v));
      }
      if (lane < LPR) {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            s_acc[(wv * GS + hh) * D + (c * LPR + j) * EPC + e] = acc[hh][c * EPC + e];
      }
      if (lane == 0) s_l[wv][hh] = lw;
    }
    __syncthreads();
    for (int i = tid; i < GS * D; i += 256) {
      const int hh = i / D, d = i - hh * D;
      const float sum = (s_acc[(0 * GS + hh) * D + d] + s_acc[(1 * GS + hh) * D + d]) +
                        (s_acc[(2 * GS + hh) * D + d] + s_acc[(3 * GS + hh) * D + d]);
      const int head = kvh * p.G + slice * GS + hh;
      const size_t o = ((size_t)b * p.Hq + head) * p.nsplit + split;
      p.pacc[o * D + d] = sum;
      if (d == 0) {
        p.pm[o] = fmaxf(fmaxf(s_m[0][hh], s_m[1][hh]), fmaxf(s_m[2][hh], s_m[3][hh]));
        p.pl[o] = (s_l[0][hh] + s_l[1][hh]) + (s_l[2][hh] + s_l[3][hh]);
      }
    }
  }
}

// One work-group of 128 threads per (head, sequence); thread d owns output
// element d. Everything that depends on nothing (the first SB splits' acc
// values, this thread's (max, sum) pair, the query row for the cache update)
// is loaded up front, so the kernel waits on memory about once.
__global__ __launch_bounds__(128) void combine_kernel(CombineParams p) {
  // thread t takes dimensions 4*(t % nq) .. +3 (nq = d/4 quads) of the splits
  // t / nq, t / nq + nsg, ... (nsg = 128 / nq split groups): 16-byte loads,
  // SB of them held in registers; the groups meet in LDS at the end
  constexpr int SB = 16;
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[4];
  __shared__ __align__(16) float s_o[4 * 128];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int ns = p.nsplit;
  const size_t base = ((size_t)b * p.Hq + h) * ns;
  const bool own_d = tid < p.d;
  const int nq = p.d >> 2, nsg = 128 / nq;
  const int dq = tid % nq, sg = tid / nq;
  const float4* pa = reinterpret_cast<const float4*>(p.pacc + base * p.d) + dq;
  float4 a[SB];
#pragma unroll
  for (int i = 0; i < SB; ++i) {
    const int s = sg + i * nsg;
    a[i] = s < ns ? pa[(size_t)s * nq] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // the cache update's inputs (decision, query element, first selection
  // entry of this head's share) are requested now, not after the merge
  const bool upd = p.cache.prev_q != nullptr;
  const int ck = upd ? p.cache.k : 0;
  const int per = upd ? (ck + p.Hq - 1) / p.Hq : 0;
  const int lo = h * per, hi = min(ck, lo + per);
  int hit = 0;
  uint32_t qbits = 0;
  int32_t sel0 = 0;
  if (upd) {
    hit = p.cache.hit[b];
    const size_t qo = ((size_t)b * p.Hq + h) * p.d + min(tid, p.d - 1);
    qbits = p.dtype == 1 ? (uint32_t)((const uint16_t*)p.q)[qo] << 16
                         : __float_as_uint(((const float*)p.q)[qo]);
    if (p.idx_out && lo + tid < hi) sel0 = p.cache.sel[(size_t)b * ck + lo + tid];
  }
  // the step's fp64 log-sum-exp sums (read by the vote kernel, which ran
  // before this one) start the next step at zero
  if (upd && p.cache.lse_sum && tid < kLseCopies) {
    p.cache.lse_sum[((size_t)b * p.Hq + h) * kLseCopies + tid] = 0.0;
    if (h == 0 && tid == 0) p.cache.lse_big[b] = 0u;
  }
  float pmv = -INFINITY, plv = 0.f;
  if (tid < ns) {
    pmv = p.pm[base + tid];
    plv = p.pl[base + tid];
  }
  // splits past 128 (long selections): folded in a loop
  float m = plv > 0.f ? pmv : -INFINITY;
  for (int s = tid + 128; s < ns; s += 128)
    if (p.pl[base + s] > 0.f) m = fmaxf(m, p.pm[base + s]);
  m = wave_max(m);
  if (lane == 0) s_red[wv] = m;
  __syncthreads();
  const float M = fmaxf(s_red[0], s_red[1]);
  float lsum = 0.f;
  if (tid < ns) {
    const float w = plv > 0.f ? ex2(pmv - M) : 0.f;
    s_w[tid] = w;
    lsum = plv * w;
  }
  for (int s = tid + 128; s < ns; s += 128) {
    const float pl = p.pl[base + s];
    const float w = pl > 0.f ? ex2(p.pm[base + s] - M) : 0.f;
    s_w[s] = w;
    lsum += pl * w;
  }
  lsum = wave_sum(lsum);
  if (lane == 0) s_red[2 + wv] = lsum;
  __syncthreads();
  const float L = s_red[2] + s_red[3];
  // every split's acc was written (zeros for an empty split, whose weight is 0)
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](const float4 (&x)[SB], int s0) {
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int s = s0 + sg + i * nsg;
      if (s < ns) {
        const float w = s_w[s];
        o.x = fmaf(x[i].x, w, o.x); o.y = fmaf(x[i].y, w, o.y);
        o.z = fmaf(x[i].z, w, o.z); o.w = fmaf(x[i].w, w, o.w);
      }
    }
  };
  add(a, 0);
  // more splits (dense attention): further register blocks of SB loads each
  for (int s0 = SB * nsg; s0 < ns; s0 += SB * nsg) {
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int s = s0 + sg + i * nsg;
      a[i] = s < ns ? pa[(size_t)s * nq] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    add(a, s0);
  }
  *reinterpret_cast<float4*>(s_o + sg * p.d + 4 * dq) = o;
  __syncthreads();
  if (own_d) {
    float sum = 0.f;
    for (int g = 0; g < nsg; ++g) sum += s_o[g * p.d + tid];
    p.out[((size_t)b * p.Hq + h) * p.d + tid] = (L > 0.f) ? sum / L : 0.f;
  }

  // Selection-Cache state update, spread over the head blocks of a sequence
  if (!upd) return;
  const SelCacheDev& c = p.cache;
  const int n = c.Hq * c.d;
  if (c.mode == 0 || !hit) {
    float* pq = c.prev_q + (size_t)b * n + (size_t)h * c.d;
    if (own_d) pq[tid] = __uint_as_float(qbits);
  }
  if (p.idx_out) {
    const int32_t* sel = c.sel + (size_t)b * c.k;
    if (lo + tid < hi) p.idx_out[(size_t)b * c.k + lo + tid] = sel0;
    for (int i = lo + tid + 128; i < hi; i += 128) p.idx_out[(size_t)b * c.k + i] = sel[i];
  }
  if (h == 0 && tid == 0) {
    c.valid[b] = p.seq_lens[b] > 0 ? 1 : 0;
    if (hit) c.hits[b] += 1;
    else c.misses[b] += 1;
    if (p.hit_out) p.hit_out[b] = hit;
  }
}

template <int DT, int D, bool PAGED, bool DENSE, bool SEL = false>
static hipError_t launch_attend_gs(const AttendParams& p, hipStream_t s) {
  dim3 grid(p.nsplit, p.Hkv * p.nslices, p.B);
  switch (p.GS) {
#define TS_GS(n) case n: TS_KLAUNCH((attend_kernel<DT, D, n, PAGED, DENSE, SEL>), grid, dim3(256), 0, s, p); break;
    TS_GS(1) TS_GS(2) TS_GS(3) TS_GS(4) TS_GS(5) TS_GS(6) TS_GS(7) TS_GS(8)
#undef TS_GS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool DENSE>
static hipError_t launch_attend_mode(int dtype, int d, bool paged, const AttendParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return paged ? launch_attend_gs<1, 128, true, DENSE>(p, s) : launch_attend_gs<1, 128, false, DENSE>(p, s);
  if (dtype == 1 && d == 64) return paged ? launch_attend_gs<1, 64, true, DENSE>(p, s) : launch_attend_gs<1, 64, false, DENSE>(p, s);
  if (dtype == 0 && d == 128) return paged ? launch_attend_gs<0, 128, true, DENSE>(p, s) : launch_attend_gs<0, 128, false, DENSE>(p, s);
  if (dtype == 0 && d == 64) return paged ? launch_attend_gs<0, 64, true, DENSE>(p, s) : launch_attend_gs<0, 64, false, DENSE>(p, s);
  return hipErrorInvalidValue;
}

// idx null: dense attention over every cached token
hipError_t launch_attend(int dtype, int d, bool paged, const AttendParams& p, hipStream_t s) {
  if (p.sel_ctrl) {   // decode step: the selection is finished by the attention work-groups
    if (dtype == 1 && d == 128) return paged ? launch_attend_gs<1, 128, true, false, true>(p, s) : launch_attend_gs<1, 128, false, false, true>(p, s);
    if (dtype == 1 && d == 64) return paged ? launch_attend_gs<1, 64, true, false, true>(p, s) : launch_attend_gs<1, 64, false, false, true>(p, s);
    if (dtype == 0 && d == 128) return paged ? launch_attend_gs<0, 128, true, false, true>(p, s) : launch_attend_gs<0, 128, false, false, true>(p, s);
    if (dtype == 0 && d == 64) return paged ? launch_attend_gs<0, 64, true, false, true>(p, s) : launch_attend_gs<0, 64, false, false, true>(p, s);
    return hipErrorInvalidValue;
  }
  return p.idx ? launch_attend_mode<false>(dtype, d, paged, p, s) : launch_attend_mode<true>(dtype, d, paged, p, s);
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  TS_KLAUNCH(combine_kernel, dim3(p.Hq, p.B), dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
