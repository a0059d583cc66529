// fa_decode.hip — incremental decode against a paged KV cache on gfx950.
//
// Page "FlashAttention 实战指南：如何把训练内存省 20 倍、速度提 4 倍", section
// "增量解码场景flash_attn_with_kvcache": each decode step appends the new K and V
// to the cache and attends in place; rotary_cos/rotary_sin apply a built-in
// rotary embedding; cache_seqlens marks each sample's valid length;
// block_table turns on a paged cache; num_splits cuts the keys into pieces
// to balance latency for small batches with long contexts.
//
// Split kernel: one work-group per (sequence, K/V head, split).  A split is a
// contiguous range of pages.  The path is bound by HBM bandwidth, so the
// kernel runs one wave per SIMD and spends its registers and LDS on bytes in
// flight.  Its 4 waves take 32-key tiles round robin, each wave streaming
// its own tiles with no work-group barrier:
//   * K and V rows go HBM -> LDS by DMA into wave-private tiles, whole
//     256-byte row pieces per lane group; K is read back in natural order as
//     the A operand of S^T = K Q^T, V transposed as the A operand of
//     O^T += V^T P^T.  (Loading K straight into VGPRs in operand order
//     fetches 32 bytes of each row per instruction, which streams from HBM
//     about a quarter slower than whole row pieces.)
//   * two stages: while a tile is computed, the next tile's K and V are in
//     flight (16 KB per wave; the LDS holds 2 stages x 4 waves x K and V);
//   * all query heads of the group (Hq / Hkv <= 32) are the 32 columns of the
//     B operand, so every K/V byte is read once for the whole group;
//   * the rotated query is split into a 16-bit high part and a 16-bit
//     remainder and both are multiplied, so rounding the rotated query to
//     16 bits costs no accuracy in the scores;
//   * the wave whose tiles include position cache_seqlens[b] rotates k_new,
//     writes it and v_new to the cache slot in its prologue and patches them
//     into that tile, so no other work-group ever reads that slot;
//   * sequences are served longest cache first, which keeps the tail short
//     when lengths differ.
// The 4 waves' (max, sum, O) states are merged exactly in LDS.  With one
// split the kernel writes the final output; otherwise it writes float32
// partials (O_s normalised, LSE_s) that the combine kernel merges with
//   M = max_s LSE_s,  LSE = M + ln sum_s e^{LSE_s - M},  O = sum_s e^{LSE_s - LSE} O_s.
#include <algorithm>
#include <mutex>

#include "fa_device.h"
#include "fa_host.h"

namespace fa {

struct DecParams {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int* cache_seqlens;
  const int* block_table;
  int max_blocks, page_size;
  const float* cos;
  const float* sin;
  int rotary_dim;
  uint16_t* out;
  float* lse;
  float* ws_o;
  float* ws_lse;
  int B, Hq, Hkv, G, num_splits;
  int T;       // new queries per sequence (Sq_new); G * T <= 32 columns
  int causal;  // with T > 1: new query t sees keys up to its own position
  int wr;      // right window (non-causal, T > 1), -1 = unbounded
  float scale_log2;
  // logit options (the OPTS kernels): softcap c (cap_log2 = c log2 e,
  // scale_over_cap = scale / c; 0 = off), ALiBi slopes per query head, and a
  // left window (-1 = unbounded)
  float cap_log2, scale_over_cap;
  const float* alibi;
  int wl;
};

template <int DT>
__device__ __forceinline__ u32x4 pack8(const float x[8]) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack2<DT>(x[2 * e], x[2 * e + 1]);
  return r;
}

template <int DT>
__device__ __forceinline__ float lo16(uint32_t v) { return to_f32<DT>((uint16_t)(v & 0xffff)); }
template <int DT>
__device__ __forceinline__ float hi16(uint32_t v) { return to_f32<DT>((uint16_t)(v >> 16)); }

typedef __attribute__((address_space(4))) const int cint;  // constant address space

// Batches up to this size are scheduled longest cache first.
constexpr int kDecodeSortMax = 64;

// The G * T new queries of a K/V head are the MFMA columns (column
// t * G + g = query head g of the group, new token t).  New token t sits at
// position n_keys - T + t (bottom-right alignment); causal limits it to the
// keys at or before that position (with T = 1 that is every key), a left
// window w to keys >= position - w.  OPTS: softcap, ALiBi or a window is on.
// With T > 1 the appended rows were written by decode_append_kernel before
// this kernel starts; with T = 1 the kernel appends in its own prologue.
// DG < D: head dim DG in memory padded to D on chip (zero fragments and tile
// columns past DG).
template <int D, int DT, bool OPTS, int DG = D>
__global__ __launch_bounds__(256, 1) void decode_split_kernel(DecParams p) {
  constexpr int BK = 32;  // keys per wave tile
  constexpr int KC = D / 16, DB = D / 32;
  constexpr int VT = BK * D * 2;  // bytes of one wave's V tile
  // vector-memory instructions per tile load: the K and the V copy
  constexpr int NVM = 2 * (VT / 1024 > 0 ? VT / 1024 : 1);
  // K and V tiles, one per wave and stage; four distinct arrays (K and V of
  // each stage) so a read of one is never ordered behind the DMA into another.
  __shared__ __attribute__((aligned(1024))) char ks0[4 * VT];
  __shared__ __attribute__((aligned(1024))) char ks1[4 * VT];
  __shared__ __attribute__((aligned(1024))) char vs0[4 * VT];
  __shared__ __attribute__((aligned(1024))) char vs1[4 * VT];
  __shared__ float mbuf[4 * 32], lbuf[4 * 32];
  __shared__ __attribute__((aligned(16))) char apbuf[4 * D];  // rotated k_new row, v_new row
  __shared__ __attribute__((aligned(16))) char qst[33 * D * 2];  // query rows (G * T <= 32), k_new row

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  const int hf = lane >> 5, r = lane & 31;
  const uint32_t tb = tr_base<D>(lane);
  const int s_id = blockIdx.x % p.num_splits;
  const int hkv = (blockIdx.x / p.num_splits) % p.Hkv;
  const int rank = blockIdx.x / (p.num_splits * p.Hkv);
  // Work-groups are dispatched roughly in id order and one fits per CU, so
  // the sequences are taken longest cache first (ties by index): the rank-th
  // id group serves the sequence whose length has that rank.  Integer work
  // only; every work-group computes the same permutation.
  __shared__ int sel_b;
  int b = rank;
  if (p.B <= kDecodeSortMax) {
    for (int bb = tid; bb < p.B; bb += 256) {
      const int lb = p.cache_seqlens[bb];
      int rk = 0;
      for (int o = 0; o < p.B; ++o) {
        const int lo = p.cache_seqlens[o];
        rk += (lo > lb) | ((lo == lb) & (o < bb));
      }
      if (rk == rank) sel_b = bb;
    }
    __syncthreads();
    b = sel_b;
  }

  // b and every index derived from it are wave-uniform; reading the cache
  // lengths and the block table through the constant address space makes
  // them scalar loads, which the vector-memory counter of the K/V stream
  // does not have to drain.
  b = __builtin_amdgcn_readfirstlane(b);
  const int L = ((const cint*)p.cache_seqlens)[b];
  const int T = p.T, G = p.G;
  const bool append = p.k_new != nullptr;
  const bool fused = append && T == 1;  // append in this kernel's prologue
  const int n_keys = L + (append ? T : 0);
  const int qpos0 = n_keys - T;  // position of new token 0
  const int page = p.page_size;
  const int n_pages = (n_keys + page - 1) / page;
  // first key any column sees; the splits share the pages from its page on
  const int key_lo = (OPTS && p.wl >= 0) ? max(0, qpos0 - p.wl) : 0;
  const int pg0 = key_lo / page;
  const int per = (n_pages - pg0 + p.num_splits - 1) / p.num_splits;
  const int p_lo = pg0 + s_id * per;
  const int p_hi = min(n_pages, p_lo + per);
  const int k_lo = max(p_lo * page, key_lo);
  const int k_hi = min(p_hi * page, n_keys);

  // ---- stage the query rows of the G * T columns and (T = 1 append) the
  // k_new row in LDS with independent loads (one round trip) ----
  constexpr int NCH = D / 8;
  const int hr = p.cos ? p.rotary_dim / 2 : 0;  // rotary half width (0 = off)
  {
    // chunks past DG / 8 are written as zeros (padded head dim)
    const int nq = G * T * NCH, nk = fused ? NCH : 0;
    for (int i = tid; i < nq + nk; i += 256) {
      if (i < nq) {
        const int row = i / NCH, ch = i % NCH;  // row = column t * G + g
        const int t = row / G, gq = row % G;
        const u32x4 v = (DG == D || ch < DG / 8)
                            ? gload128(p.q + (((int64_t)b * T + t) * p.Hq + hkv * G + gq) * DG + ch * 8)
                            : u32x4{0, 0, 0, 0};
        lds_write128(qst, (row * D + ch * 8) * 2, v);
      } else {
        const int ch = i - nq;
        const u32x4 v = (DG == D || ch < DG / 8) ? gload128(p.k_new + ((int64_t)b * p.Hkv + hkv) * DG + ch * 8)
                                                 : u32x4{0, 0, 0, 0};
        lds_write128(qst, (32 * D + ch * 8) * 2, v);
      }
    }
    zero_pad<D, 4 * BK, DG>(ks0, tid, 256);
    zero_pad<D, 4 * BK, DG>(ks1, tid, 256);
    zero_pad<D, 4 * BK, DG>(vs0, tid, 256);
    zero_pad<D, 4 * BK, DG>(vs1, tid, 256);
    __syncthreads();
  }
  // Chunk ch (8 elements) of a staged row, rotated at position pos: the
  // half-split pairs (x_i, x_{i+hr}) for i < hr; dims >= 2 hr pass through.
  auto rot8 = [&](const char* row, int ch, int pos, float x[8]) {
    const u32x4 a = lds_read128(row, ch * 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = lo16<DT>(a[e]);
      x[2 * e + 1] = hi16<DT>(a[e]);
    }
    const int d0 = 8 * ch;
    if (d0 < 2 * hr) {
      const bool first = d0 < hr;
      const int pch = first ? ch + hr / 8 : ch - hr / 8;
      const int fi0 = first ? d0 : d0 - hr;
      const u32x4 bv = lds_read128(row, pch * 16);
      const float* cr = p.cos + (int64_t)pos * hr + fi0;
      const float* sr = p.sin + (int64_t)pos * hr + fi0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = (e & 1) ? hi16<DT>(bv[e >> 1]) : lo16<DT>(bv[e >> 1]);
        const float c = cr[e], sn = sr[e];
        x[e] = first ? (x[e] * c - y * sn) : (x[e] * c + y * sn);
      }
    }
  };

  // ---- query fragment (B operand, column = new token t, query head g) ----
  const bool col_ok = r < G * T;
  const int col_t = col_ok ? r / G : 0;
  const int qpos = qpos0 + col_t;                   // this column's query position
  // last key it sees (a right bound only binds with T > 1)
  const int right = p.causal ? 0 : p.wr;
  const int last_key = right >= 0 ? min(n_keys - 1, qpos + right) : n_keys - 1;
  const int first_key = (OPTS && p.wl >= 0) ? max(0, qpos - p.wl) : 0;
  u32x4 qhi[KC], qlo[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (col_ok) {
      float x[8], rem[8];
      rot8(qst + r * (D * 2), 2 * c + hf, L + col_t, x);
      qhi[c] = pack8<DT>(x);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rem[2 * e] = x[2 * e] - lo16<DT>(qhi[c][e]);
        rem[2 * e + 1] = x[2 * e + 1] - hi16<DT>(qhi[c][e]);
      }
      qlo[c] = pack8<DT>(rem);
    } else {
      qhi[c] = u32x4{0, 0, 0, 0};
      qlo[c] = u32x4{0, 0, 0, 0};
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) oacc[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float slope_log2 = (OPTS && p.alibi && col_ok) ? p.alibi[hkv * G + r % G] * kLog2e : 0.0f;

  // Element offset of the first row of the 32-key tile starting at key j0
  // (a tile never crosses a page: page_size is a multiple of 32).  Rows of
  // a tile are Hkv * D elements apart.
  const int64_t cap = (int64_t)p.max_blocks * page;
  auto tile_base = [&](int j0) -> int64_t {
    if (p.block_table) {
      const int phys = ((const cint*)p.block_table)[(int64_t)b * p.max_blocks + j0 / page];
      return (((int64_t)phys * page + (j0 % page)) * p.Hkv + hkv) * DG;
    }
    return (((int64_t)b * cap + j0) * p.Hkv + hkv) * DG;
  };
  const int64_t kvstride = (int64_t)p.Hkv * DG;

  // Tiles of this split, dealt round robin to the 4 waves.
  const int t_lo = k_lo / BK, t_hi = (k_hi + BK - 1) / BK;
  const int t_first = t_lo + w;
  const int n_my = (k_lo < k_hi && t_first < t_hi) ? (t_hi - t_first + 3) / 4 : 0;

  // K and V rows of tile t go by DMA into this wave's LDS tiles.
  auto load = [&](int t, char* kdst, char* vdst) {
    const int64_t base = tile_base(t * BK);
    dma_tile<D, BK, 1, true, DG>(kdst, p.k_cache + base, kvstride, 0, BK, 0, lane);
    dma_tile<D, BK, 1, true, DG>(vdst, p.v_cache + base, kvstride, 0, BK, 0, lane);
  };
  const uint32_t nb = nat_base<D>(lane);

  // One tile: `kt` / `vt` hold K and V of tile t.
  auto compute = [&](int t, char* kt, char* vt) {
    const int j0 = t * BK;
    if (fused && L >= j0 && L < j0 + BK) {
      // This tile holds the appended position: its row takes the rotated
      // k_new and v_new parked in LDS by the prologue instead of the stale
      // cache row that was streamed in (the lanes of that row write it and
      // are the ones that read its K fragments; LDS accesses of a wave are
      // ordered, so the transposed V reads see it too).
      if (r == L - j0) {
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          lds_write128(kt, tile_off<D>(r, 2 * c + hf), lds_read128(apbuf, (2 * c + hf) * 16));
          lds_write128(vt, tile_off<D>(r, 2 * c + hf), lds_read128(apbuf + 2 * D, (2 * c + hf) * 16));
        }
      }
    }
    if (j0 + BK > n_keys && r >= n_keys - j0) {
      // Rows past the last key hold whatever the page holds there (never
      // written, recycled, or the pre-append slot of a later call); their
      // weights are 0, but 0 * inf or 0 * NaN in P V would not be, so their
      // V rows are zeroed (their logits are masked below).
#pragma unroll
      for (int c = 0; c < KC; ++c) lds_write128(vt, tile_off<D>(r, 2 * c + hf), u32x4{0, 0, 0, 0});
    }
    u32x4 ka[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = lds_nat(kt, nb, c);
    // two independent accumulation chains (high and low query part): one
    // wave per SIMD has no other wave to hide a single chain's MFMA latency
    f32x16 s = f32x16{}, sl = f32x16{};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      s = mfma32<DT>(ka[c], qhi[c], s);
      sl = mfma32<DT>(ka[c], qlo[c], sl);
    }
    s += sl;
    if constexpr (OPTS) {
      // final logits in log2 units: softcap, then the ALiBi distance term
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = p.cap_log2 > 0.0f ? p.cap_log2 * tanh_exp(s[i] * p.scale_over_cap) : s[i] * p.scale_log2;
        if (p.alibi) x -= slope_log2 * (float)abs(qpos - (j0 + frag_row(i, hf)));
        s[i] = x;
      }
    }
    // keys past a column's own position (causal, T > 1), past the cache end,
    // or left of its window are masked
    const int min_last = right >= 0 ? min(n_keys - 1, qpos0 + right) : n_keys - 1;
    const int max_first = (OPTS && p.wl >= 0) ? qpos0 + T - 1 - p.wl : 0;
    if (j0 + BK - 1 > min_last || (OPTS && j0 < max_first)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = j0 + frag_row(i, hf);
        s[i] = (j <= last_key && j >= first_key) ? s[i] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = pair_max32(mx);
    if constexpr (!OPTS) mx *= p.scale_log2;
    if (__any(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int d = 0; d < DB; ++d) oacc[d] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = fast_exp2(fmaf(s[i], OPTS ? 1.0f : p.scale_log2, -m_use));
      s[i] = pv;
      lsum += pv;
    }
    l_run += lsum;
#pragma unroll
    for (int mk = 0; mk < 2; ++mk) {
      const u32x4 pb = pack_frag_half<DT>(s, mk);
#pragma unroll
      for (int d = 0; d < DB; ++d) oacc[d] = mfma32<DT>(lds_At<D>(vt + (16 * mk) * (D * 2), tb, d), pb, oacc[d]);
    }
  };

  // Append (once per call): the wave whose tiles include position L rotates
  // k_new, writes the rotated key and v_new to the cache slot (no other
  // wave or work-group reads that slot) and parks both rows in LDS for the
  // tile that uses them.
  if (fused && L >= k_lo && L < k_hi && ((L / BK - t_lo) & 3) == w && r == L % BK) {
    const uint16_t* vnr = p.v_new + ((int64_t)b * p.Hkv + hkv) * DG;
    const int64_t slot = tile_base(L - L % BK) + (int64_t)r * kvstride;
    u32x4 vv[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const bool in = DG == D || (2 * c + hf) * 8 < DG;
      vv[c] = in ? gload128(vnr + (2 * c + hf) * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      float x[8];
      rot8(qst + 32 * (D * 2), 2 * c + hf, L, x);
      const u32x4 kk = pack8<DT>(x);
      if (DG == D || (2 * c + hf) * 8 < DG) {
        gstore128(p.k_cache + slot + (2 * c + hf) * 8, kk);
        gstore128(p.v_cache + slot + (2 * c + hf) * 8, vv[c]);
      }
      lds_write128(apbuf, (2 * c + hf) * 16, kk);
      lds_write128(apbuf + 2 * D, (2 * c + hf) * 16, vv[c]);
    }
  }
  // (the stores above retire before the stream's first wait; they are older
  // than every tile load)

  // Two-stage stream: while tile i is computed, tile i+1 is in flight.
  // VMEM operations retire in order, so waiting until only the next tile's
  // NVM operations are outstanding completes tile i.  The copy into a stage
  // is issued after the previous use of that stage has been computed (its
  // LDS reads have returned: the MFMAs consumed them).
  char* kt0 = ks0 + w * VT;
  char* kt1 = ks1 + w * VT;
  char* vt0 = vs0 + w * VT;
  char* vt1 = vs1 + w * VT;
  auto stage = [&](int i, char* kc, char* vc, char* kn, char* vn) {
    const int t = t_first + 4 * i;
    if (i + 1 < n_my) load(t + 4, kn, vn);
    asm volatile("" ::: "memory");
    if (i + 1 < n_my) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NVM));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    compute(t, kc, vc);
  };
  if (n_my > 0) load(t_first, kt0, vt0);
  for (int i = 0; i < n_my; i += 2) {
    stage(i, kt0, vt0, kt1, vt1);
    if (i + 1 < n_my) stage(i + 1, kt1, vt1, kt0, vt0);
  }

  // ---- merge the 4 waves: M = max m_w, each wave scaled by 2^(m_w - M) ----
  const float l_w = pair_sum32(l_run);
  if (hf == 0) {
    mbuf[w * 32 + r] = m_run;
    lbuf[w * 32 + r] = l_w;
  }
  __syncthreads();  // also ends every wave's use of its V tiles
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mbuf[ww * 32 + r]);
  const float M_use = (M == -INFINITY) ? 0.0f : M;
  const float fw = (m_run == -INFINITY) ? 0.0f : fast_exp2(m_run - M_use);
  // O^T fragments accumulate into obuf[d][32] (float), one wave after another
  float* obuf = reinterpret_cast<float*>(vs0);
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) {
          const int dd = 32 * d + frag_row(i2, hf);
          const float v = oacc[d][i2] * fw;
          obuf[dd * 32 + r] = (ww == 0) ? v : obuf[dd * 32 + r] + v;
        }
    }
    __syncthreads();
  }
  // ---- write: each thread handles (column, d) pairs ----
  for (int idx = tid; idx < G * T * DG; idx += 256) {
    const int col = idx / DG, d = idx % DG;
    const int h = hkv * G + col % G, tt = col / G;
    const int64_t bht = ((int64_t)b * p.Hq + h) * T + tt;  // (b, h, t) of lse and partials
    float Mc = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) Mc = fmaxf(Mc, mbuf[ww * 32 + col]);
    const float Mcu = (Mc == -INFINITY) ? 0.0f : Mc;
    float lc = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = mbuf[ww * 32 + col];
      lc += (mw == -INFINITY) ? 0.0f : lbuf[ww * 32 + col] * fast_exp2(mw - Mcu);
    }
    const float o = lc > 0.0f ? obuf[d * 32 + col] / lc : 0.0f;
    if (p.num_splits == 1) {
      uint16_t* orow = p.out + (((int64_t)b * T + tt) * p.Hq + h) * DG;
      const uint32_t pk = pack2<DT>(o, 0.0f);
      orow[d] = (uint16_t)(pk & 0xffff);
      if (d == 0 && p.lse) p.lse[bht] = lc > 0.0f ? (Mc + fast_log2(lc)) * kLn2 : INFINITY;
    } else {
      const int64_t pi = bht * p.num_splits + s_id;
      p.ws_o[pi * DG + d] = o;
      if (d == 0) p.ws_lse[pi] = lc > 0.0f ? (Mc + fast_log2(lc)) * kLn2 : -INFINITY;
    }
  }
}

// One wave per (sequence, query head):
//   M = max_s LSE_s,  LSE = M + ln sum_s e^{LSE_s - M},  O = sum_s e^{LSE_s - LSE} O_s.
// Lane s holds split s's weight (splits taken 64 at a time), broadcast by
// shuffles; each lane accumulates output elements d = lane and lane + 64
// with the partial loads unrolled so several are in flight.
template <int D, int DT>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecParams p) {
  const int bh = blockIdx.x;  // (b * Hq + h) * T + t
  const int lane = threadIdx.x;
  const int S = p.num_splits;
  const float* ls = p.ws_lse + (int64_t)bh * S;
  const float* os = p.ws_o + (int64_t)bh * S * D;
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, ls[s]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  const float Mu = (M == -INFINITY) ? 0.0f : M;
  float sum = 0.0f;
  for (int s = lane; s < S; s += 64) sum += fast_exp2((ls[s] - Mu) * kLog2e);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  const bool empty = !(sum > 0.0f);
  const float L = empty ? INFINITY : Mu + fast_log2(sum) * kLn2;
  constexpr int ND = (D + 63) / 64;
  float o[ND];
#pragma unroll
  for (int k = 0; k < ND; ++k) o[k] = 0.0f;
  if (!empty) {
    for (int s0 = 0; s0 < S; s0 += 64) {
      const int ns = min(64, S - s0);
      const float wl = lane < ns ? fast_exp2((ls[s0 + lane] - L) * kLog2e) : 0.0f;
      int s = 0;
      for (; s + 8 <= ns; s += 8) {
        float part[8][ND];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int k = 0; k < ND; ++k) {
            const int d = lane + 64 * k;
            part[u][k] = d < D ? os[(int64_t)(s0 + s + u) * D + d] : 0.0f;
          }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wgt = __shfl(wl, s + u, 64);
#pragma unroll
          for (int k = 0; k < ND; ++k) o[k] = fmaf(wgt, part[u][k], o[k]);
        }
      }
      for (; s < ns; ++s) {
        const float wgt = __shfl(wl, s, 64);
#pragma unroll
        for (int k = 0; k < ND; ++k) {
          const int d = lane + 64 * k;
          if (d < D) o[k] = fmaf(wgt, os[(int64_t)(s0 + s) * D + d], o[k]);
        }
      }
    }
  }
  // out is (B, T, Hq, D); bh = (b * Hq + h) * T + t
  const int tt = bh % p.T, h = (bh / p.T) % p.Hq, b = bh / (p.T * p.Hq);
  uint16_t* orow = p.out + (((int64_t)b * p.T + tt) * p.Hq + h) * D;
#pragma unroll
  for (int k = 0; k < ND; ++k) {
    const int d = lane + 64 * k;
    if (d < D) {
      const uint32_t pk = pack2<DT>(o[k], 0.0f);
      orow[d] = (uint16_t)(pk & 0xffff);
    }
  }
  if (lane == 0 && p.lse) p.lse[bh] = L;
}

// Append for T > 1 new tokens, launched before the split kernel: one wave
// per (sequence, new token, K/V head) rotates k_new at position
// cache_seqlens[b] + t (half-split pairs, caller's tables), rounds it once to
// the cache dtype and writes it and v_new to the token's cache slot.  The
// split kernel then reads the slots like any other cache row.
template <int D, int DT>
__global__ __launch_bounds__(256) void decode_append_kernel(DecParams p) {
  constexpr int NCH = D / 8;
  const int id = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (id >= p.B * p.T * p.Hkv || lane >= NCH) return;
  const int hkv = id % p.Hkv, t = (id / p.Hkv) % p.T, b = id / (p.Hkv * p.T);
  const int pos = p.cache_seqlens[b] + t;
  int64_t slot;
  if (p.block_table) {
    const int phys = p.block_table[(int64_t)b * p.max_blocks + pos / p.page_size];
    slot = (((int64_t)phys * p.page_size + pos % p.page_size) * p.Hkv + hkv) * D;
  } else {
    slot = (((int64_t)b * p.max_blocks * p.page_size + pos) * p.Hkv + hkv) * D;
  }
  const int64_t src = (((int64_t)b * p.T + t) * p.Hkv + hkv) * D;
  const int ch = lane, d0 = 8 * ch;
  const int hr = p.cos ? p.rotary_dim / 2 : 0;
  const u32x4 a = gload128(p.k_new + src + d0);
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = lo16<DT>(a[e]);
    x[2 * e + 1] = hi16<DT>(a[e]);
  }
  if (d0 < 2 * hr) {
    const bool first = d0 < hr;
    const int pd = first ? d0 + hr : d0 - hr;  // partner chunk
    const int fi0 = first ? d0 : d0 - hr;
    const u32x4 bv = gload128(p.k_new + src + pd);
    const float* cr = p.cos + (int64_t)pos * hr + fi0;
    const float* sr = p.sin + (int64_t)pos * hr + fi0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y = (e & 1) ? hi16<DT>(bv[e >> 1]) : lo16<DT>(bv[e >> 1]);
      x[e] = first ? (x[e] * cr[e] - y * sr[e]) : (x[e] * cr[e] + y * sr[e]);
    }
  }
  gstore128(p.k_cache + slot + d0, pack8<DT>(x));
  gstore128(p.v_cache + slot + d0, gload128(p.v_new + src + d0));
}

// D: head dim on chip; DG: in memory (96 runs padded on the 128 kernel)
template <int D, int DT, int DG = D>
static int launch_decode(const DecParams& p, bool opts, hipStream_t st) {
  const long long nwg = (long long)p.B * p.Hkv * p.num_splits;
  if (nwg > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  if (p.k_new && p.T > 1) {
    const long long rows = (long long)p.B * p.T * p.Hkv;
    hipLaunchKernelGGL((decode_append_kernel<DG, DT>), dim3((int)((rows + 3) / 4)), dim3(256), 0, st, p);
  }
  prof_before(FA_KERNEL_DECODE_SPLIT, st);
  if (opts) hipLaunchKernelGGL((decode_split_kernel<D, DT, true, DG>), dim3((int)nwg), dim3(256), 0, st, p);
  else hipLaunchKernelGGL((decode_split_kernel<D, DT, false, DG>), dim3((int)nwg), dim3(256), 0, st, p);
  prof_after(FA_KERNEL_DECODE_SPLIT, st);
  if (p.num_splits > 1) {
    prof_before(FA_KERNEL_DECODE_COMBINE, st);
    hipLaunchKernelGGL((decode_combine_kernel<DG, DT>), dim3(p.B * p.Hq * p.T), dim3(64), 0, st, p);
    prof_after(FA_KERNEL_DECODE_COMBINE, st);
  }
  return launch_status();
}

// num_splits = 0 lets the library choose.  The split kernel holds one
// work-group per CU (256 CUs), and an HBM-bound stream wants several rounds
// of them in flight, so the choice aims at about 1024 work-groups, with at
// most kAutoSplitMax splits and no more splits than pages.
constexpr int kAutoSplitMax = 32;
constexpr int kAutoTargetGroups = 1024;

static int auto_splits(int B, int Hkv, int max_pages) {
  const long long groups = (long long)B * Hkv;
  long long s = (kAutoTargetGroups + groups - 1) / groups;
  s = std::min<long long>(s, kAutoSplitMax);
  s = std::min<long long>(s, max_pages);
  return (int)std::max<long long>(s, 1);
}

// ------------------------------------------------- no-allocation variant --
// Split partials of fa_fwd_kvcache_noalloc live in this file-scope device
// array, one copy per GPU, held until the process ends.  Host code never
// uses its name as an address (on the host it is only a stand-in symbol):
// the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch` (NULL on error).
static void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace fa

using namespace fa;

extern "C" size_t fa_kvcache_workspace_size(int B, int Sq_new, int Hq, int D, int num_splits) {
  if (num_splits == 0) num_splits = kAutoSplitMax;  // enough for any automatic choice
  if (B < 1 || Sq_new < 1 || Hq < 1 || D < 1 || num_splits <= 1) return 0;
  const size_t parts = (size_t)B * Sq_new * Hq * num_splits;
  return align_up(parts * D * sizeof(float), 256) + align_up(parts * sizeof(float), 256);
}

extern "C" int fa_fwd_kvcache(const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, const int* cache_seqlens,
                              const int* block_table, int max_blocks_per_seq, int page_size,
                              const float* rotary_cos, const float* rotary_sin, int rotary_dim,
                              void* out, float* lse,
                              int B, int Sq_new, int Hq, int Hkv, int D, int dtype,
                              float scale, int causal, int window_left, int window_right, float softcap,
                              const float* alibi_slopes, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_common(Hq, Hkv, D, dtype, scale, window_left, window_right, softcap);
  if (st) return st;
  if (B < 1 || Sq_new < 1 || num_splits < 0 || max_blocks_per_seq < 1) return FA_ERR_INVALID_ARG;
  if (page_size < 32 || page_size % 32 != 0) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return FA_ERR_INVALID_ARG;
  if (!aligned4(cache_seqlens)) return FA_ERR_INVALID_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return FA_ERR_INVALID_ARG;
  if (!opt_aligned16(k_new) || !opt_aligned16(v_new)) return FA_ERR_INVALID_ARG;
  if (block_table && !aligned4(block_table)) return FA_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return FA_ERR_INVALID_ARG;
  if ((rotary_cos == nullptr) != (rotary_sin == nullptr)) return FA_ERR_INVALID_ARG;
  if (rotary_cos && (rotary_dim < 16 || rotary_dim % 16 != 0 || rotary_dim > D)) return FA_ERR_INVALID_ARG;
  if (rotary_cos && (!aligned4(rotary_cos) || !aligned4(rotary_sin))) return FA_ERR_INVALID_ARG;
  if (alibi_slopes && !aligned4(alibi_slopes)) return FA_ERR_INVALID_ARG;
  // D = 256: two stages of a wave's private 32-key K and V tiles would take
  // 64 KB per wave, 256 KB for the four waves of a work-group (LDS: 160 KB)
  if (D == 256) return FA_ERR_UNSUPPORTED;
  // the G * Sq_new new queries of a K/V head are the 32 MFMA columns
  if ((long long)(Hq / Hkv) * Sq_new > 32) return FA_ERR_UNSUPPORTED;
  if (num_splits == 0) num_splits = auto_splits(B, Hkv, max_blocks_per_seq);
  const size_t need = fa_kvcache_workspace_size(B, Sq_new, Hq, D, num_splits);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return FA_ERR_WORKSPACE;

  DecParams p{};
  p.q = (const uint16_t*)q;
  p.k_new = (const uint16_t*)k_new;
  p.v_new = (const uint16_t*)v_new;
  p.k_cache = (uint16_t*)k_cache;
  p.v_cache = (uint16_t*)v_cache;
  p.cache_seqlens = cache_seqlens;
  p.block_table = block_table;
  p.max_blocks = max_blocks_per_seq;
  p.page_size = page_size;
  p.cos = rotary_cos;
  p.sin = rotary_sin;
  p.rotary_dim = rotary_cos ? rotary_dim : 0;
  p.out = (uint16_t*)out;
  p.lse = lse;
  const size_t parts = (size_t)B * Sq_new * Hq * num_splits;
  p.ws_o = need ? (float*)workspace : nullptr;
  p.ws_lse = need ? (float*)((char*)workspace + align_up(parts * D * sizeof(float), 256)) : nullptr;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.num_splits = num_splits;
  p.T = Sq_new;
  p.causal = causal ? 1 : 0;
  p.wr = window_right;
  p.scale_log2 = scale * kLog2e;
  p.cap_log2 = softcap * kLog2e;
  p.scale_over_cap = softcap > 0.0f ? scale / softcap : 0.0f;
  p.alibi = alibi_slopes;
  p.wl = window_left;
  // one new query at the last position sees every earlier key, so only a
  // left window, softcap or ALiBi changes the scores
  const bool opts = softcap > 0.0f || alibi_slopes != nullptr || window_left >= 0;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = dtype == FA_DTYPE_BF16;
  switch (D) {
    case 32: return bf ? launch_decode<32, DT_BF16>(p, opts, s) : launch_decode<32, DT_F16>(p, opts, s);
    case 64: return bf ? launch_decode<64, DT_BF16>(p, opts, s) : launch_decode<64, DT_F16>(p, opts, s);
    case 96: return bf ? launch_decode<128, DT_BF16, 96>(p, opts, s) : launch_decode<128, DT_F16, 96>(p, opts, s);
    case 128: return bf ? launch_decode<128, DT_BF16>(p, opts, s) : launch_decode<128, DT_F16>(p, opts, s);
    default: return FA_ERR_UNSUPPORTED;
  }
}

extern "C" size_t fa_kvcache_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int fa_fwd_kvcache_noalloc(const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache, const int* cache_seqlens,
                                      const int* block_table, int max_blocks_per_seq, int page_size,
                                      const float* rotary_cos, const float* rotary_sin, int rotary_dim,
                                      void* out, float* lse,
                                      int B, int Sq_new, int Hq, int Hkv, int D, int dtype,
                                      float scale, int causal, int window_left, int window_right,
                                      float softcap, const float* alibi_slopes, int num_splits, void* stream) {
  if (B < 1 || Sq_new < 1 || Hq < 1 || Hkv < 1 || D < 1 || num_splits < 0 || max_blocks_per_seq < 1)
    return FA_ERR_INVALID_ARG;
  const int ns = num_splits == 0 ? auto_splits(B, Hkv, max_blocks_per_seq) : num_splits;
  const size_t need = fa_kvcache_workspace_size(B, Sq_new, Hq, D, ns);
  if (need > kScratchBytes) return FA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_ptr();
    if (!ws) return FA_ERR_LAUNCH;
  }
  return fa_fwd_kvcache(q, k_new, v_new, k_cache, v_cache, cache_seqlens, block_table, max_blocks_per_seq,
                        page_size, rotary_cos, rotary_sin, rotary_dim, out, lse, B, Sq_new, Hq, Hkv, D, dtype,
                        scale, causal, window_left, window_right, softcap, alibi_slopes, ns, ws, kScratchBytes,
                        stream);
}
