// Live Pipeline fused step: the predictor of layer l + 1 runs while layer l's sparse
// up and down rows are gathered (KAIROX page, Core method, item 2: the attention
// output of layer i feeds the predictor of layer i + 1, overlapped with layer i's
// FFN; Key observation 1: adjacent layers' hidden states have cosine similarity
// about 0.98, so one layer ahead keeps the prediction close).
//
// Each layer j has two inputs: x_j, the FFN input, and xp_j, the predictor input
// (a caller that pipelines a real model passes xp_j = x_{j-1}, available when layer
// j - 1 starts; NULL means x_j).  Per layer, exactly what sfx_ffn_step computes,
// except that the scores, masks and list come from xp_j:
//   scores_j = W2 relu(W1 xp_j),  list_j = ascending {i : score >= t} (union over
//   tokens),  hact = act(Wa[i] x_j + b_i),  y_j = sum hact Wd[i].
//
// Schedule (one workgroup of 512 threads per compute unit, all resident):
//   prologue   predictor of layer 0 (hidden, scores, union exchange, list)
//   layer l    gather waves (0..3 and 7): hidden of layer l + 1 (waves 0..3, W1 row
//              in registers), the Wd segments and the up rows of layer l's list,
//              activations out, down -> y_l; then the union exchange of layer l + 1
//              and the scan that builds its list in LDS.
//              stream waves (4..6): wait for layer l + 1's W2 rows in LDS (issued one
//              layer earlier), read the hidden, score, union words out, then issue
//              the W2 rows of layer l + 2.
//              grid barrier (layer l + 1's input depends on y_l through attention)
// The stream waves take no gathers: a wave's loads complete in issue order, so
// loads issued behind a 40 KB W2 share would wait for it.
//
// Hand-offs are k_step's tagged words, with the tag of the layer they belong to:
// hidden and union words of layer l + 1 are written after the barrier of layer l - 1,
// when every reader of layer l's words (the scores and union exchange of layer l,
// both before that barrier) is done.
#pragma once
#include "k_step.hpp"

namespace sfx {
namespace step {

constexpr int kNG = kAW + 1;             // gather waves: 0..kAW-1 and kCW
constexpr int kNS = kCW - kAW;           // stream waves: kAW..kCW-1
constexpr int kSpRed = kRedFloats / 2;   // s_red: [0, kSpRed) scores of own rows, then the down sums
#ifndef SFX_PIPE_PRED_PRIO
#define SFX_PIPE_PRED_PRIO 3
#endif
constexpr int kPredPrio = SFX_PIPE_PRED_PRIO;   // wave issue priority (s_setprio) of the predictor work

// gather slot of a wave: kCW -> 0 (free at the start of a layer), waves 0..kAW-1 -> 1..kAW
__device__ __forceinline__ int gather_slot(int wave) { return wave == kCW ? 0 : wave + 1; }

// Bytes of the hidden staging area at the end of s_x (the list of the layer being
// gathered sits before it and stays live meanwhile).
__host__ __device__ constexpr int pipe_hid_bytes(int TB, int h) { return 4 * TB * h; }

template <class T, int NB, bool REGLU, int DL>
__global__ __launch_bounds__(kNT, 1) void k_pipe(StepParams p) {
  constexpr int kU = 8 * DL;
  constexpr int TB = NB < 4 ? NB : 4;
  constexpr int kUP = (NB == 1 && !REGLU) ? kU : (NB == 1 || (NB == 2 && !REGLU)) ? 4 : 2;
  constexpr int kRD = NB == 1 ? 12 : NB == 2 ? 6 : 3;   // down rows per lane loaded together
  // poll back-off (x 64 clocks): re-polls of uncached words compete with the weight
  // streams; measured on the OPT-6.7B shape, 2 -> 30 took the layer period from
  // 28.1 to 25.6 us (8: 27.0, 100: 27.3); for the hidden poll alone 2 and 8 were
  // also slower (24.7, 24.2 against 23.7 us)
  constexpr int kPS = 30;
  // The hidden exchange: each workgroup's tagged hidden words packed at 4 NB words
  // (32 bytes at one token), so a round of polls over all workgroups touches a
  // quarter of the cache lines it did at 16 words.  The stream waves start polling
  // only once this workgroup's own hidden rows are out, plus a pause of kHidPause x
  // 64 clocks (the others land over about a microsecond after it): polls issued
  // before the hidden exists only added traffic.  Measured (one token, us per
  // layer-step, OPT-6.7B / LLaMA2-7B shapes): polling from the stream waves' start
  // 23.8 / 28.4; after the own hidden 21.3 / 25.9, with the pause 21.5 / 24.8;
  // packed words, after the own hidden 20.8 / 25.0, with the pause 20.9 / 24.4.
  constexpr int kHS = 4 * NB;
  constexpr int kHidPause = 40;
  constexpr int kRB = TB <= 2 ? 8 : 4;
  __shared__ __attribute__((aligned(16))) uint8_t s_w2[kW2Bytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kXBytes];
  __shared__ __attribute__((aligned(16))) float s_red[kRedFloats];
  __shared__ uint32_t s_words[64];
  __shared__ uint32_t s_wt[kNW];
  __shared__ uint32_t s_gsync, s_ssync;      // arrivals of the gather / stream waves
  __shared__ uint32_t s_hdone;               // waves 0..kAW-1 done with a round of hidden rows
  __shared__ uint32_t s_nosplit;             // = layer tag: a hidden value is outside the fp16 range
  uint32_t* s_pref = reinterpret_cast<uint32_t*>(s_x);
  uint32_t* s_uw = reinterpret_cast<uint32_t*>(s_x + kPrefBytes);
  int32_t* s_nid = reinterpret_cast<int32_t*>(s_x + kPrefBytes + kUwBytes);
  float* s_hid = reinterpret_cast<float*>(s_x + kXBytes - pipe_hid_bytes(TB, p.h));
  const int nid_cap = (kXBytes - kPrefBytes - kUwBytes - pipe_hid_bytes(TB, p.h)) / 4;
  // ReGLU up rows read the input from LDS (s_xk, below the stream waves' hidden)
  // when the layer's list leaves room for it: loaded by waves 0..3 right after the
  // list is built, waited for before the grid barrier.  Measured, one token: ReGLU
  // (two weight rows per input read) 24.2 -> 22.7 us per layer-step at the LLaMA2-7B
  // shape; ReLU 20.4 -> 21.3 at the OPT-6.7B shape (the gather waves then reach
  // the union poll earlier and their polls meet the stream waves' W2 traffic), so
  // ReLU keeps reading the input from memory.
  const long long xk_end = (long long)kXBytes - pipe_hid_bytes(TB, p.h);
  const long long xk_off = (xk_end - (long long)p.B * p.d * 2) & ~255LL;
  const int nid_cap_x = xk_off > kPrefBytes + kUwBytes ? (int)((xk_off - kPrefBytes - kUwBytes) / 4) : -1;
  uint8_t* const s_xk = s_x + (xk_off > 0 ? xk_off : 0);
  bool x_in_lds = false;
  constexpr bool kXK = REGLU;

  if (threadIdx.x == 0) { s_gsync = 0u; s_ssync = 0u; s_nosplit = 0u; s_hdone = 0u; }
  lds_barrier();
  const uint32_t e0 = ld_agent(p.fbar + (size_t)blockIdx.x * kFS);
  uint32_t gsn = 0, ssn = 0;                 // group-sync arrivals so far (wave-uniform)
  auto gather_sync = [&]() { gsn += kNG; group_sync(&s_gsync, gsn, p.err); };
  auto stream_sync = [&]() { ssn += kNS; group_sync(&s_ssync, ssn, p.err); };

  // ------------------------------------------------ predictor pieces of layer j
  // Hidden rows w + P s (waves 0..kAW-1, W1 row in registers) from the predictor
  // input, tagged out.
  Raw<16> w1r[kU];
  auto hidden = [&](CLayer* Lj, uint32_t tg) __attribute__((always_inline)) {
    SFX_PHASE_IDS;
    const int a_row = w + P * wave;
    if (!(wave < kAW && wave < p.nr1 && a_row < h)) return;
    const uint8_t* x = (const uint8_t*)(Lj->xp != nullptr ? Lj->xp : Lj->x);
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
    constexpr int MG = NB == 1 ? kU : NB == 2 ? (kU >= 4 ? kU / 2 : kU) : (kU >= 8 ? kU / 4 : kU);
#pragma unroll
    for (int m0 = 0; m0 < kU; m0 += MG) {
      Raw<16> xv[MG][NB];
#pragma unroll
      for (int i = 0; i < MG; ++i) {
        const int c = min(lane + (m0 + i) * kWave, nch1 - 1);
#pragma unroll
        for (int b = 0; b < NB; ++b) xv[i][b] = load_raw<16>(x + (size_t)min(b, B - 1) * rb1 + (size_t)c * 16);
      }
#pragma unroll
      for (int i = 0; i < MG; ++i)
        if (lane + (m0 + i) * kWave < nch1) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            if (b < B) dot_chunk<T>(w1r[m0 + i].w, xv[i][b].w, acc[b]);
        }
    }
    const float v = wave_reduce_multi<NB>(acc);
    const int b = reduce_index<NB>(lane);
    if (reduce_owner<NB>(lane) && b < B)
      st_tagged(p.hid + (size_t)w * kHS + wave * NB + b, tg, __float_as_uint(fmaxf(v, 0.f)));
  };

  // Scores of the owned rows (stream waves): wait for this wave's W2 rows, read the
  // hidden of every workgroup, score from LDS (or memory), ballots, union words
  // tagged out, outputs.
  auto scores = [&](CLayer* Lj, uint32_t tg) __attribute__((always_inline)) {
    SFX_PHASE_IDS;
    const int st = tid - kAW * kWave;        // 0 .. kNS*64-1
    constexpr int kST = kNS * kWave;
    const int nw2 = w < W ? (W - w + P - 1) / P : 0;
    const int rows2 = nw2 * 32;
    const bool w2_lds = p.w2_lds != 0;
    const uint8_t* W2 = (const uint8_t*)Lj->W2;
    float* s_sc = s_red;                     // [rows2][NB]
    if (w2_lds) wait_memory();               // this wave's LDS rows have landed
    // At one token thread st polls the blocks of workgroups st and st + kST (P <=
    // 2 kST) in one round.  With fp16 W2 rows in LDS the hidden goes in as two fp16 pieces, hi =
    // fp16(h) and lo = fp16((h - hi) 2^11), for the dot-product scores; a value
    // outside the fp16 range sends the layer to the fp32 spread and sums.
    constexpr bool kSplitH = std::is_same<T, TF16>::value;
    uint16_t* s_hh = reinterpret_cast<uint16_t*>(s_hid);   // [TB][h] hi
    uint16_t* s_hl = s_hh + (size_t)TB * h;                 // [TB][h] lo * 2^11
    auto put = [&](bool split_in, int at, float v) {
      if (split_in) {
        if (!(fabsf(v) < 65504.f)) s_nosplit = tg;
        const _Float16 hi = (_Float16)v;
        const _Float16 lo = (_Float16)((v - (float)hi) * 2048.f);
        s_hh[at] = __builtin_bit_cast(uint16_t, hi);
        s_hl[at] = __builtin_bit_cast(uint16_t, lo);
      } else {
        s_hid[at] = v;
      }
    };
    auto spread = [&](bool split_in) {
      if constexpr (NB > 1) {                // one block per poll round (register budget)
#pragma unroll 1
        for (int o = st; o < P; o += kST) {
          const int ns = o < h ? (h - o + P - 1) / P : 0;
          unsigned long long hw[4 * NB];
          auto valid = [&](int i) { return i / NB < ns && i % NB < B; };
          auto addr = [&](int i) { return p.hid + (size_t)o * kHS + i; };
          poll_tagged_if<4 * NB, decltype(valid), decltype(addr), kPS>(hw, valid, addr, tg, p.err);
#pragma unroll
          for (int i = 0; i < 4 * NB; ++i)
            if (valid(i)) put(split_in, (i % NB) * h + o + P * (i / NB), __uint_as_float((uint32_t)hw[i]));
        }
      } else if (st < P) {
        const int o1 = st, o2 = st + kST;
        const int ns1 = o1 < h ? (h - o1 + P - 1) / P : 0;
        const int ns2 = o2 < P && o2 < h ? (h - o2 + P - 1) / P : 0;
        unsigned long long hw[8 * NB];
        // entries [0, 4 NB): block o1, [4 NB, 8 NB): block o2; entry s NB + b = row o + P s, token b
        auto valid = [&](int i) {
          const int e = i % (4 * NB);
          return e / NB < (i < 4 * NB ? ns1 : ns2) && e % NB < B;
        };
        auto addr = [&](int i) {
          const int o = i < 4 * NB ? o1 : min(o2, P - 1);
          return p.hid + (size_t)o * kHS + i % (4 * NB);
        };
        poll_tagged_if<8 * NB, decltype(valid), decltype(addr), kPS>(hw, valid, addr, tg, p.err);
#pragma unroll
        for (int i = 0; i < 8 * NB; ++i) {
          if (valid(i)) {
            const int e = i % (4 * NB);
            const int o = i < 4 * NB ? o1 : o2;
            put(split_in, (e % NB) * h + o + P * (e / NB), __uint_as_float((uint32_t)hw[i]));
          }
        }
      }
      stream_sync();
    };
    const bool split_try = kSplitH && w2_lds;
    // round tg - e0 of the hidden rows: this workgroup's are out, the others' follow
    lds_wait_at_least(&s_hdone, kAW * (tg - e0), p.err);
    __builtin_amdgcn_s_sleep(kHidPause);
    spread(split_try);
    const bool split = split_try && s_nosplit != tg;
    if (split_try && !split) spread(false);   // the words are still in place: no wait
    auto pass = [&](auto from_lds) {
      constexpr bool kLds = decltype(from_lds)::value;
      for (int q0 = wave - kAW; q0 < rows2; q0 += kNS * kRB) {
        float a2[kRB * TB];
#pragma unroll
        for (int i = 0; i < kRB * TB; ++i) a2[i] = 0.f;
        for (int c = lane; c < nch2; c += kWave) {
          float hv[TB][8];
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            const float4* hp = reinterpret_cast<const float4*>(s_hid + (b < B ? b : 0) * h + c * 8);
            const float4 u0 = hp[0], u1 = hp[1];
            hv[b][0] = u0.x; hv[b][1] = u0.y; hv[b][2] = u0.z; hv[b][3] = u0.w;
            hv[b][4] = u1.x; hv[b][5] = u1.y; hv[b][6] = u1.z; hv[b][7] = u1.w;
          }
          Raw<16> wv[kRB];
#pragma unroll
          for (int r = 0; r < kRB; ++r) {
            const int q = min(q0 + r * kNS, rows2 - 1);
            if constexpr (kLds) {
              wv[r] = *reinterpret_cast<const Raw<16>*>(s_w2 + ((size_t)q * nch2 + c) * 16);
            } else {
              const int row = min(32 * (w + P * (q >> 5)) + (q & 31), f - 1);
              wv[r] = load_raw<16>(W2 + (size_t)row * rb2 + (size_t)c * 16);
            }
          }
          float wf[kRB][8];
#pragma unroll
          for (int r = 0; r < kRB; ++r) unpack<T, 4>(wv[r].w, wf[r]);
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int r = 0; r < kRB; ++r)
#pragma unroll
              for (int b = 0; b < TB; ++b) a2[r * TB + b] = fmaf(wf[r][e], hv[b][e], a2[r * TB + b]);
        }
        const float v = wave_reduce_multi<kRB * TB>(a2);
        if (reduce_owner<kRB * TB>(lane)) {
          const int ix = reduce_index<kRB * TB>(lane);
          const int r = ix / TB, b = ix - r * TB;
          const int q = q0 + r * kNS;
          if (q < rows2 && b < B) s_sc[q * NB + b] = v;
        }
      }
    };
    // the split hidden against the fp16 rows in LDS: hi and lo dot-product sums per
    // row (lo scaled back by 2^-11 at the end)
    auto pass_split = [&]() {
      for (int q0 = wave - kAW; q0 < rows2; q0 += kNS * kRB) {
        float a2[kRB * TB], a3[kRB * TB];
#pragma unroll
        for (int i = 0; i < kRB * TB; ++i) { a2[i] = 0.f; a3[i] = 0.f; }
        for (int c = lane; c < nch2; c += kWave) {
          half2_t hh[TB][4], hl[TB][4];
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            const uint4 u = *reinterpret_cast<const uint4*>(s_hh + (size_t)(b < B ? b : 0) * h + c * 8);
            const uint4 v = *reinterpret_cast<const uint4*>(s_hl + (size_t)(b < B ? b : 0) * h + c * 8);
            hh[b][0] = __builtin_bit_cast(half2_t, u.x); hh[b][1] = __builtin_bit_cast(half2_t, u.y);
            hh[b][2] = __builtin_bit_cast(half2_t, u.z); hh[b][3] = __builtin_bit_cast(half2_t, u.w);
            hl[b][0] = __builtin_bit_cast(half2_t, v.x); hl[b][1] = __builtin_bit_cast(half2_t, v.y);
            hl[b][2] = __builtin_bit_cast(half2_t, v.z); hl[b][3] = __builtin_bit_cast(half2_t, v.w);
          }
          Raw<16> wv[kRB];
#pragma unroll
          for (int r = 0; r < kRB; ++r) {
            const int q = min(q0 + r * kNS, rows2 - 1);
            wv[r] = *reinterpret_cast<const Raw<16>*>(s_w2 + ((size_t)q * nch2 + c) * 16);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < kRB; ++r) {
              const half2_t wj = __builtin_bit_cast(half2_t, wv[r].w[j]);
#pragma unroll
              for (int b = 0; b < TB; ++b) {
                a2[r * TB + b] = __builtin_amdgcn_fdot2(wj, hh[b][j], a2[r * TB + b], false);
                a3[r * TB + b] = __builtin_amdgcn_fdot2(wj, hl[b][j], a3[r * TB + b], false);
              }
            }
        }
#pragma unroll
        for (int i = 0; i < kRB * TB; ++i) a2[i] = fmaf(a3[i], 1.f / 2048.f, a2[i]);
        const float v = wave_reduce_multi<kRB * TB>(a2);
        if (reduce_owner<kRB * TB>(lane)) {
          const int ix = reduce_index<kRB * TB>(lane);
          const int r = ix / TB, b = ix - r * TB;
          const int q = q0 + r * kNS;
          if (q < rows2 && b < B) s_sc[q * NB + b] = v;
        }
      }
    };
    if (split) pass_split();
    else if (w2_lds) pass(std::true_type{});
    else pass(std::false_type{});
    stream_sync();
    const float thr = Lj->threshold;
    for (int m0 = 2 * (wave - kAW); m0 < nw2; m0 += 2 * kNS) {
      const int m = m0 + (lane >> 5);
      const int g = w + P * m;
      const int row = 32 * g + (lane & 31);
      const bool in = m < nw2 && row < f;
      for (int b = 0; b < B; ++b) {
        const uint64_t bal = __ballot(in && s_sc[(32 * m + (lane & 31)) * NB + b] >= thr);
        if ((lane & 31) == 0 && m < nw2) {
          const uint32_t word = (uint32_t)(lane == 0 ? bal : (bal >> 32));
          if (Lj->tok_bits != nullptr) Lj->tok_bits[(size_t)b * W + g] = word;
          s_words[m * NB + b] = word;
        }
      }
    }
    stream_sync();
    if (st < nw2) {
      uint32_t u = 0;
      for (int b = 0; b < B; ++b) u |= s_words[st * NB + b];
      const int g = w + P * st;
      // word-major (word m of owner o at m P + o): a poll of all owners' words is
      // nw2 P / 16 cache lines, not one per owner (20.7 -> 20.4 us, OPT-6.7B shape)
      st_tagged(p.uni + (size_t)st * P + w, tg, u);
      Lj->union_bits[g] = u;
    }
    for (int i = st; i < rows2 * B; i += kST) {
      const int q = i / B, b = i - q * B;
      const int row = 32 * (w + P * (q >> 5)) + (q & 31);
      if (row < f) Lj->scores[(size_t)b * f + row] = s_sc[q * NB + b];
    }
    stream_sync();                           // s_w2 and s_sc consumed
  };

  // Union exchange and scan (gather waves): the ascending list of layer j lands in
  // LDS (s_nid when it fits, else found from s_pref / s_uw); returns its length.
  auto union_scan = [&](CLayer* Lj, uint32_t tg) __attribute__((always_inline)) -> int {
    SFX_PHASE_IDS;
    const int gs = gather_slot(wave);
    const int gt = gs * kWave + lane;        // 0 .. kNG*64-1
    constexpr int kGT = kNG * kWave;
#pragma unroll 1
    for (int o = gt; o < P; o += kGT) {
      const int nw = o < W ? (W - o + P - 1) / P : 0;
#pragma unroll 1
      for (int m0 = 0; m0 < nw; m0 += 8) {
        unsigned long long uv[8];
        const int n = min(8, nw - m0);
        auto valid = [&](int i) { return i < n; };
        auto addr = [&](int i) { return p.uni + (size_t)(m0 + i) * P + o; };
        poll_tagged_if<8, decltype(valid), decltype(addr), kPS>(uv, valid, addr, tg, p.err);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < n) s_uw[o + P * (m0 + i)] = (uint32_t)uv[i];
      }
    }
    gather_sync();
    // thread gt owns words [wpt gt, wpt gt + wpt)
    const int wpt = (W + kGT - 1) / kGT;
    const int g0 = wpt * gt;
    uint32_t cnt = 0;
    for (int g = g0; g < min(W, g0 + wpt); ++g) cnt += __popc(s_uw[g]);
    const uint32_t inc = wave_inclusive_scan_u32(cnt);
    if (lane == kWave - 1) s_wt[gs] = inc;
    gather_sync();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int v = 0; v < kNG; ++v) {
      const uint32_t t = s_wt[v];
      if (v < gs) before += t;
      total += t;
    }
    uint32_t pos = before + inc - cnt;
    const int k = (int)total;
    const bool in_lds = k <= nid_cap;
    for (int g = g0; g < min(W, g0 + wpt); ++g) {
      s_pref[g] = pos;
      pos += __popc(s_uw[g]);
    }
    if (gt == 0) s_pref[W] = total;
    if (w == 0 && gt == 0) *Lj->count = k;
    gather_sync();
    // the list, one byte of a word per step, bytes interleaved over the threads, so
    // the dense words of hot-first storage spread over many threads
    if (in_lds) {
      for (int bt = gt; bt < 4 * W; bt += kGT) {
        const int g = bt >> 2, sh = 8 * (bt & 3);
        const uint32_t word = s_uw[g];
        uint32_t wd = (word >> sh) & 0xFFu;
        uint32_t at = s_pref[g] + __popc(word & ((1u << sh) - 1u));
        while (wd) { s_nid[at++] = 32 * g + sh + __builtin_ctz(wd); wd &= wd - 1; }
      }
    }
    gather_sync();
    return k;
  };

  // ------------------------------------------------ FFN of layer l (gather waves)
  // One up row: Wa (and Wl) row of neuron nid against x, bias, activation; out
  // tagged by neuron for the down phase, and at rank r in the outputs.
  auto up_row = [&](CLayer* Ld, int nid, int r, uint32_t tg) __attribute__((always_inline)) {
    SFX_PHASE_IDS;
    const uint8_t* x = (const uint8_t*)Ld->x;
    const uint8_t* ra = (const uint8_t*)Ld->Wa + (size_t)nid * rb1;
    const uint8_t* rl = REGLU ? (const uint8_t*)Ld->Wl + (size_t)nid * rb1 : nullptr;
    const float bias = Ld->ba != nullptr ? Ld->ba[nid] : 0.f;
    float za[NB], zl[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) { za[b] = 0.f; zl[b] = 0.f; }
#pragma unroll
    for (int u0 = 0; u0 < kU; u0 += kUP) {
      Raw<16> wa[kUP], wl[kUP], xq[kUP][NB];
#pragma unroll
      for (int u = 0; u < kUP; ++u) {
        const int c = min(lane + (u0 + u) * kWave, nch1 - 1);
        wa[u] = load_raw<16>(ra + (size_t)c * 16);
        if (REGLU) wl[u] = load_raw<16>(rl + (size_t)c * 16);
      }
      if (x_in_lds) {
#pragma unroll
        for (int u = 0; u < kUP; ++u)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            xq[u][b] = *reinterpret_cast<const Raw<16>*>(s_xk + (size_t)min(b, B - 1) * rb1 +
                                                         (size_t)min(lane + (u0 + u) * kWave, nch1 - 1) * 16);
      } else {
#pragma unroll
        for (int u = 0; u < kUP; ++u)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            xq[u][b] = load_raw<16>(x + (size_t)min(b, B - 1) * rb1 + (size_t)min(lane + (u0 + u) * kWave, nch1 - 1) * 16);
      }
#pragma unroll
      for (int u = 0; u < kUP; ++u) {
        if (lane + (u0 + u) * kWave < nch1) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            if (b < B) {
              dot_chunk<T>(wa[u].w, xq[u][b].w, za[b]);
              if (REGLU) dot_chunk<T>(wl[u].w, xq[u][b].w, zl[b]);
            }
        }
      }
    }
    const float ta = wave_reduce_multi<NB>(za);
    float v = fmaxf(ta + bias, 0.f);
    if (REGLU) v *= wave_reduce_multi<NB>(zl);
    if (reduce_owner<NB>(lane)) {
      const int b = reduce_index<NB>(lane);
      if (b < B) {
        st_tagged(p.hact + (size_t)nid * B + b, tg, __float_as_uint(v));
        Ld->hact[(size_t)r * B + b] = v;
      }
    }
    if (lane == 0) Ld->idx[r] = nid;
  };

  // ------------------------------------------------ prologue: layer 0's predictor
  CLayer* L0 = (CLayer*)p.layers;
  prefetch_w1<kU>(p, L0, w1r);
  prefetch_w2(p, L0, s_w2);
  int k = 0;
  {
    int wave = threadIdx.x >> 6;
    asm volatile("" : "+v"(wave));
    const uint32_t tg0 = e0 + 1u;
    if (wave < kAW) {
      hidden(L0, tg0);
      group_arrive(&s_hdone);
    }
    if (wave >= kAW && wave < kCW) {
      scores(L0, tg0);
      if (p.L > 1) prefetch_w2(p, L0 + 1, s_w2);
    } else {
      k = union_scan(L0, tg0);
      x_in_lds = kXK && k <= nid_cap_x;
      if (x_in_lds && wave < kAW) {
        load_x_lds(p, L0, s_xk);
        wait_memory();
      }
      gather_sync();
      if (wave < kAW && p.L > 1) prefetch_w1<kU>(p, L0 + 1, w1r);
    }
  }

  for (int l = 0; l < p.L; ++l) {
    const uint32_t tag = e0 + (uint32_t)l + 1u;
    CLayer* Ld = (CLayer*)p.layers + l;
    const bool has_next = l + 1 < p.L;
    int wave = threadIdx.x >> 6;
    asm volatile("" : "+v"(wave));
    if (wave >= kAW && wave < kCW) {
      // ---------------------------------------------------- stream waves
      if (has_next) {
        // the next layer's predictor is the critical path: its waves take issue
        // priority over the gathers on the shared SIMDs while they score
        __builtin_amdgcn_s_setprio(kPredPrio);
        scores(Ld + 1, tag + 1u);
        __builtin_amdgcn_s_setprio(0);
        if (l + 2 < p.L) prefetch_w2(p, Ld + 2, s_w2);
      }
    } else {
      // ---------------------------------------------------- gather waves
      SFX_PHASE_IDS;
      const bool in_lds = k <= nid_cap;
      const int gs = gather_slot(wave);
      // hidden of the next layer first (its W1 row is in registers; the input is
      // in memory since the layer started)
      if (has_next && wave < kAW) {
        __builtin_amdgcn_s_setprio(kPredPrio);
        hidden(Ld + 1, tag + 1u);
        group_arrive(&s_hdone);
        __builtin_amdgcn_s_setprio(0);
      }
      // down geometry: lane group j = lane mod nct reads columns c0 + 8 j; slot
      // gs * 64/nct + lane / nct walks the list
      const int nct = p.cw / 8;
      const int d_tile = tile_of(w, P);
      const int c0 = d_tile * p.cw;
      const int d_j = lane & (nct - 1);
      const int d_rr = gs * (kWave / nct) + lane / nct;
      const int d_rs = kNG * (kWave / nct);
      const int d_col = c0 + d_j * 8;
      const bool d_ok = d_col < d;
      const uint8_t* Wd = (const uint8_t*)Ld->Wd;
      Raw<16> wdv[kRD];
      int nid[kRD];
      auto nid_of = [&](int r) { return in_lds ? s_nid[r] : rank_to_neuron(r, s_pref, s_uw, W); };
      auto load_wd = [&](int rb) {
#pragma unroll
        for (int u = 0; u < kRD; ++u) nid[u] = nid_of(min(rb + u * d_rs, k - 1));
#pragma unroll
        for (int u = 0; u < kRD; ++u) wdv[u] = load_raw<16>(Wd + (size_t)nid[u] * rb1 + (size_t)d_col * 2);
      };
      // up rows of this workgroup's share of the list: ranks [r0, r1), row i of the
      // share to gather slot i mod kNG; then the first batch of Wd segments
      // (measured: up rows before the segments 28.9 -> 28.0 us per layer)
      {
        const int r0 = (int)(((long long)k * w) / P), r1 = (int)(((long long)k * (w + 1)) / P);
        for (int r = r0 + gs; r < r1; r += kNG) up_row(Ld, nid_of(r), r, tag);
      }
      if (d_ok && d_rr < k) load_wd(d_rr);
      // down: activations by neuron (tagged), fixed-order sums -> y columns
      float yacc[NB * 8];
#pragma unroll
      for (int i = 0; i < NB * 8; ++i) yacc[i] = 0.f;
      if (d_ok) {
        for (int rb = d_rr; rb < k; rb += d_rs * kRD) {
          if (rb != d_rr) load_wd(rb);
          unsigned long long hv[kRD * NB];
          const int nrow = min(kRD, (k - rb + d_rs - 1) / d_rs);
          auto valid = [&](int i) { return i / NB < nrow && i % NB < B; };
          auto addr = [&](int i) { return p.hact + (size_t)nid[i / NB] * B + min(i % NB, B - 1); };
          poll_tagged_if<kRD * NB, decltype(valid), decltype(addr), kPS>(hv, valid, addr, tag, p.err);
#pragma unroll
          for (int u = 0; u < kRD; ++u) {
            if (u < nrow) {
              float wf[8];
              unpack<T, 4>(wdv[u].w, wf);
#pragma unroll
              for (int b = 0; b < NB; ++b)
                if (b < B) {
                  const float hvf = __uint_as_float((uint32_t)hv[u * NB + b]);
#pragma unroll
                  for (int e = 0; e < 8; ++e) yacc[b * 8 + e] = fmaf(hvf, wf[e], yacc[b * 8 + e]);
                }
            }
          }
        }
      }
      constexpr int V = NB * 8;
      const float v = wave_reduce_multi_groups<V, 2>(yacc);
      float* s_dred = s_red + kSpRed;        // [kNG][64]
      if ((lane & (kWave / V - 1)) < 2) s_dred[gs * 64 + (lane >> (6 - ilog2c(V))) * 2 + (lane & 1)] = v;
      gather_sync();                         // down sums in; the list of layer l is consumed
      const int gt = gs * kWave + lane;
      for (int i = gt; i < nct * B * 8; i += kNG * kWave) {
        const int j = i / (B * 8);
        const int be = i - j * B * 8;
        const int col = c0 + j * 8 + (be & 7);
        if (col < d) {
          float s = 0.f;
          for (int g2 = 0; g2 < kNG; ++g2)
            for (int jj = j; jj < 2; jj += nct) s += s_dred[g2 * 64 + be * 2 + jj];
          Ld->y[(size_t)(be >> 3) * d + col] = s;
        }
      }
      if (has_next) {
        k = union_scan(Ld + 1, tag + 1u);    // its first sync also orders the s_dred reads
        x_in_lds = kXK && k <= nid_cap_x;
        if (x_in_lds && wave < kAW) load_x_lds(p, Ld + 1, s_xk);
        if (wave < kAW && l + 2 < p.L) prefetch_w1<kU>(p, Ld + 2, w1r);
      }
    }
    if (has_next) {
      // grid barrier: every workgroup raises its flag once its layer is done
      if (x_in_lds && wave < kAW) wait_memory();
      lds_barrier();
      if (threadIdx.x == 0) store_through(p.fbar + (size_t)blockIdx.x * kFS, tag);
      if (wave == kCW) wait_flags(p.fbar, gridDim.x, tag, p.err, 1u);
      lds_barrier();
    }
  }
  if (threadIdx.x == 0) store_through(p.fbar + (size_t)blockIdx.x * kFS, e0 + (uint32_t)p.L);
}

template <class T, int NB, int DL>
hipError_t run_pipe(hipStream_t s, const StepParams& p, int act, int P) {
  if (act == 1) k_pipe<T, NB, true, DL><<<dim3(P), dim3(kNT), 0, s>>>(p);
  else k_pipe<T, NB, false, DL><<<dim3(P), dim3(kNT), 0, s>>>(p);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch_pipe(hipStream_t s, const StepParams& p, int act, int P) {
  switch (nb_class(p.B)) {
    case 1: return run_pipe<T, 1, 1>(s, p, act, P);
    case 2: return run_pipe<T, 2, 1>(s, p, act, P);
    default: return run_pipe<T, 4, 1>(s, p, act, P);
  }
}

template <class T, int NB, int DL>
int pipe_blocks(int act) {
  int n = 0;
  hipError_t e = act == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pipe<T, NB, true, DL>, kNT, 0)
                          : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pipe<T, NB, false, DL>, kNT, 0);
  return e == hipSuccess ? n : 0;
}
template <class T>
int pipe_blocks_per_cu(int act, int B) {
  switch (nb_class(B)) {
    case 1: return pipe_blocks<T, 1, 1>(act);
    case 2: return pipe_blocks<T, 2, 1>(act);
    default: return pipe_blocks<T, 4, 1>(act);
  }
}

}  // namespace step
}  // namespace sfx
