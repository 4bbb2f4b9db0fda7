// Forward kernels: exact attention with online softmax, gfx950.
//
// One workgroup owns one tile of 256 queries of one (batch, head) and streams
// the key/value tiles past it (the flipped loop order of "Flash Attention,
// From First Principles", "The schedule -- who commutes?": the query block is
// resident, its output is written once).  Each of the 8 waves owns 32 query
// rows.  Per key tile a wave
//   1. mints the score tile on the matrix cores, transposed: S^T = K Q^T, so
//      each lane holds the scores of ONE query against 16 keys and its partner
//      lane (32 away) the other 16 ("The scaffold": S_tile = Q_tile K_tile^T);
//   2. masks keys past the end and, on diagonal tiles, keys after the
//      query's last visible key;
//   3. forms P = exp(S - m) against its running max m, adds the row sums to
//      the running sum l and rounds P to bf16; when a tile would push some p
//      past a fixed bound, m first moves to the true running max and l and
//      the accumulator are rescaled by exp(m_old - m_new) ("LLM Architecture
//      Refresh [3]", sections 2 and 4);
//   4. accumulates O^T += V^T P^T on the matrix cores -- the bf16 P registers
//      are already in the B-operand layout, no data movement;
// and after the last tile divides once by l and stores O and the
// log-sum-exp ("FlashAttention from scratch", Step 3 and Follow-up questions).
// Key tiles lying wholly after the workgroup's last query are skipped
// ("LLM Architecture Refresh [3]", section 7).
//
// Schedule: the waves form two groups of four, one wave of each group per
// SIMD.  In every round one group issues only matrix-core work (the value
// product of the previous tile and the scores of the current one) while the
// other runs the softmax of its scores on the vector ALUs, then the groups
// swap; a workgroup barrier separates the halves.  So each SIMD keeps its
// matrix core and its vector ALU busy with two waves whose own instruction
// streams need not interleave the two kinds of work.
//
// Scores are kept in log2 units: t = s * c - m with c = |scale| * log2(e), so
// each probability costs one FMA and one v_exp_f32.  A negative scale is
// handled by negating the query fragment (exact in bf16/fp32).
//
// K and V tiles go from HBM straight into LDS by DMA (global_load_lds), two
// stages deep.  Both tiles stay row-major in LDS (XOR-swizzled against bank
// conflicts); the V^T operand of the PV product is read with the transposing
// ds_read_b64_tr_b16, so no register shuffling is needed.
//
// That is the head-dimension-128 kernel (fwd_bf16_kernel).  The same steps run
// in: fwd_inorder_kernel (d = 64: 128-query tiles, every wave in order, four
// workgroups per CU), fwd_d256_kernel and fwd_d256_pair_kernel (d = 256; the
// second for causal grids of one wave: balanced pairs of query tiles),
// fwd_fp8_kernel (e4m3 inputs), fwd_decode_kernel (a few query rows per key /
// value head, keys split and merged by fwd_merge_kernel), fwd_f32_kernel and,
// for grids too small to fill the GPU, fwd_f32_split_kernel (fp32 inputs).
#include <algorithm>
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

// Eight waves in two groups of four; the hardware places wave w on SIMD
// w % 4, so every SIMD runs one wave of each group.
constexpr int kWaves = 8;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
static_assert(kBM == fwd_rows_per_tile(128), "plan geometry");
// The fp32 kernel keeps the 4-wave, 128-query tiling.
constexpr int kWavesF32 = 4;
constexpr int kBMF32 = 32 * kWavesF32;

// A tile's probabilities are accepted against the running max m as it stands
// as long as every lane's sum of p stays <= kSumBound (so every p <= 2^8);
// otherwise the tile rebases m to the true running max first.
constexpr float kSumBound = 256.f;
// Start value of the running max (log2 units): finite, so exp2(t - m) is +inf
// (never NaN) for every finite score of the first tile, which forces a rebase.
constexpr float kMInit = -1e30f;

template <int D, int BN>
struct FwdCfg {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per tile row
  static constexpr int TILE_BYTES = BN * D * 2;     // one K or V tile (bf16)
  static constexpr int OFF_V = 2 * TILE_BYTES;      // K[2] at 0, V[2] at OFF_V
  static constexpr int OFF_Q = 4 * TILE_BYTES;      // the workgroup's query tile
  static constexpr int Q_BYTES = kBM * D * 2;
  static constexpr int SMEM_BYTES = OFF_Q + Q_BYTES;
  static constexpr int QDMA = Q_BYTES / (1024 * kWaves);     // query-tile DMAs per wave
  static constexpr int NSB = BN / 32;               // 32-key sub-blocks per tile
  static constexpr int NQC = D / 16;                // 16-feature chunks (QK^T k-steps)
  static constexpr int NDB = D / 32;                // 32-feature output blocks
  static constexpr int DMA = TILE_BYTES / (16 * 64 * kWaves);  // DMAs per lane per tile
  static constexpr int DMA_STRIDE = 16 * 64 * kWaves;          // bytes between them
  static constexpr int ROW_BYTES = CPR * 16;
  static_assert(DMA * DMA_STRIDE == TILE_BYTES, "tile split");
  static_assert(Q_BYTES == 4 * TILE_BYTES, "the output tile fits the K/V stages");
};

// Per-lane byte offset (inside one (batch, head) slice, relative to row k0) of
// the global chunk that lands in this lane's LDS slot of DMA number i.  Rows
// past N are clamped to row N-1 (finite data; those keys are masked to -inf
// and their P is 0, so they contribute nothing).  Both the LDS tile and the
// global rows are D * 2 bytes long, so with either swizzle DMA i + 1 is DMA i
// shifted by DMA_STRIDE bytes on both sides (for a full tile).
template <int D, int BN, int KIND>
__device__ __forceinline__ unsigned dma_src_off(int i, int w, int lane, int k0, int N, bool full) {
  using C = FwdCfg<D, BN>;
  const int slot = (i * kWaves + w) * 64 + lane;
  const int row = slot / C::CPR;
  const int chunk = (slot % C::CPR) ^ swz<C::CPR, KIND>(row);
  const int src_row = full ? row : min(k0 + row, N - 1) - k0;
  return (unsigned)((src_row * D + chunk * 8) * 2);
}

// Workgroup barrier that orders the compiler's memory operations but adds no
// wait for outstanding memory transfers (prefetch DMAs stay in flight).
__device__ __forceinline__ void phase_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Problem of one launch.  Nq query rows against Nk keys per head; with causal
// masking query i sees key j iff j <= i + koff (koff = Nk - Nq: the queries
// are the last Nq positions).  The keys may be split into nsplit ranges of
// klen keys, one workgroup per (query tile, range); each range's normalised
// output and log-sum-exp go to Opart / Lpart (fp32) for fwd_merge_kernel.
struct FwdArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* LSE;
  float* Opart;   // [nsplit, BH, Nq, D] when nsplit > 1
  float* Lpart;   // [nsplit, BH, Nq]
  int BH, Nq, Nk, koff, nqt, nsplit, klen, group, negq;
  float c;
  int prio1, prio2, prio3;   // remaining-round thresholds of the issue priorities
  int pass;                  // compute units per XCD (the snake order's period)
};

template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_bf16_kernel(const FwdArgs a) {
  const uint16_t* __restrict__ Q = a.Q;
  const uint16_t* __restrict__ K = a.K;
  const uint16_t* __restrict__ V = a.V;
  const int BH = a.BH, Nq = a.Nq, Nk = a.Nk, koff = a.koff, group = a.group;
  const float c = a.c;
  using C = FwdCfg<D, BN>;
  constexpr int NSB = C::NSB;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2;            // 0: matrix phase first; 1: softmax phase first
  const int n = lane & 31;
  const int h = lane >> 5;

  int bh, qt, sp = 0;
  {
    int bid = blockIdx.x;
    if (a.nsplit > 1) {
      sp = bid % a.nsplit;
      bid /= a.nsplit;
    }
    map_tile(bid, BH, a.nqt, CAUSAL, &bh, &qt);
  }
  const size_t base = (size_t)bh * (size_t)Nq * D;
  // grouped-query attention: `group` consecutive query heads share one key /
  // value head (1 for plain multi-head attention); the grid order keeps the
  // query heads of a group on one XCD whenever the heads per XCD allow
  const size_t kvbase = (size_t)(bh / group) * (size_t)Nk * D;
  const uint16_t* Qh = Q + base;
  const char* Kb = reinterpret_cast<const char*>(K + kvbase);
  const char* Vb = reinterpret_cast<const char*>(V + kvbase);

  // 32-query blocks alternate between the groups so both see the same share
  // of the causal diagonal.
  const int q0 = qt * kBM;
  const int wq0 = q0 + 32 * (2 * (w & 3) + grp);   // this wave's first query
  const int qrow = wq0 + n;                        // this lane's query

  // this workgroup's keys: [kb, ke), cut at the tile's last visible key
  const int kb = sp * a.klen;
  int ke = min(Nk, kb + a.klen);
  if (CAUSAL) ke = min(ke, q0 + kBM + koff);
  const int nkt = ke > kb ? (ke - kb + BN - 1) / BN : 0;

  // DMA: tile t of K (V) goes to K (V) stage t & 1.  Round j issues K tile
  // j + 1 and V tile j; they land by the end of round j and are read in round
  // j + 1 (K by the scores of tile j + 1, V by the value product of tile j).
  // Each tile is issued at the start of a softmax phase, never during a
  // matrix phase (a DMA instruction costs about 16 cycles at the CU's address
  // unit; a burst of them held back the other group's matrix work): group 1
  // issues K tile j + 1 as round j begins, group 0 issues V tile j when its
  // softmax half of round j begins (V stage j & 1 was last read in round
  // j - 1).  Each wave fills two 1 KiB slots per DMA step of its tile.
  const unsigned ldsb = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
  const int ws0 = w & 3, ws1 = ws0 + 4;   // the two DMA slots a wave fills
  const unsigned koffA = dma_src_off<D, BN, SWZ_ROWS>(0, ws0, lane, 0, Nk, true);
  const unsigned voffA = dma_src_off<D, BN, SWZ_TR>(0, ws0, lane, 0, Nk, true);
  const unsigned koffB = dma_src_off<D, BN, SWZ_ROWS>(0, ws1, lane, 0, Nk, true);
  const unsigned voffB = dma_src_off<D, BN, SWZ_TR>(0, ws1, lane, 0, Nk, true);
  auto issue_slot = [&](int t, int ws, unsigned lds_tensor, const char* gsrc, unsigned off0,
                        auto kind) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kind)::value;
    const int k0 = kb + t * BN;
    const char* g = gsrc + (size_t)k0 * D * 2;
    const unsigned st = ldsb + ws * 1024 + lds_tensor + (t & 1) * C::TILE_BYTES;
    if (k0 + BN <= Nk) {
#pragma unroll
      for (int i = 0; i < C::DMA; ++i)
        dma16(g + i * C::DMA_STRIDE, off0, st + i * C::DMA_STRIDE);
    } else {
#pragma unroll
      for (int i = 0; i < C::DMA; ++i)
        dma16(g, dma_src_off<D, BN, KIND>(i, ws, lane, k0, Nk, false), st + i * C::DMA_STRIDE);
    }
  };
  auto issue = [&](int t, unsigned lds_tensor, const char* gsrc, unsigned offA, unsigned offB,
                   auto kind) __attribute__((always_inline)) {
    issue_slot(t, ws0, lds_tensor, gsrc, offA, kind);
    issue_slot(t, ws1, lds_tensor, gsrc, offB, kind);
  };
  using rows_t = std::integral_constant<int, SWZ_ROWS>;
  using tr_t = std::integral_constant<int, SWZ_TR>;
  if (nkt > 0 && grp == 1) issue(0, 0u, Kb, koffA, koffB, rows_t{});

  // The query tile (kBM rows) goes HBM -> LDS by DMA in whole 1 KiB rows
  // (row swizzle, as K) and from there into registers: per-lane 16-byte
  // loads straight from HBM would touch 32 rows per instruction.  Wave w
  // fills slots w, w + 8, ..; DMA i + 1 is DMA i shifted by 8 KiB on both
  // sides, which keeps the swizzle (a multiple of 16 rows).  Rows past Nq
  // fall outside the buffer resource and read 0.
  {
    const int slot = w * 64 + lane;
    const int row = slot / C::CPR;
    const int chunk = (slot % C::CPR) ^ swz<C::CPR, SWZ_ROWS>(row);
    const unsigned qoff = (unsigned)((row * D + chunk * 8) * 2);
    const long long qbytes = (long long)max(0, Nq - q0) * (D * 2);
#pragma unroll
    for (int i = 0; i < C::QDMA; ++i) {
      const long long b0 = (long long)i * 1024 * kWaves;
      const long long nrec = qbytes - b0 > 0 ? qbytes - b0 : 0;
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(reinterpret_cast<const char*>(Qh + (size_t)q0 * D) + b0), (short)0, (int)nrec,
          0x00020000);
      dma16_buf(rsrc, qoff, ldsb + C::OFF_Q + (unsigned)b0 + w * 1024);
    }
  }
  // this wave's 32 query rows inside the workgroup's tile
  const int wblk = 2 * (w & 3) + grp;
  bf16x8 qf[C::NQC];   // Q^T B operands, read from the query tile below

  // Per-lane LDS operand addresses inside a stage, one register per tensor.
  // K (A operand of S^T): row 32sb + n, features 16cc + 8h..  With the row
  // swizzle the chunk is (2cc + h) ^ (n % 16), so the byte offset is
  // ka ^ (32 cc) with ka the cc = 0 offset: the XOR only touches bits 5..7,
  // the sub-block and stage offsets are added as immediates.
  const int ka = tile_off<C::CPR, SWZ_ROWS>(n, 8 * h);
  // V^T (A operand of O^T += V^T P^T) through transposing reads: 16-lane group
  // g reads key rows 4*(g/2) + j (+16kc, +8 for the second half) and features
  // 32db + 16*(g%2) + 4*(lane%4).  With the transposing swizzle (chunk ^ 4(r%4))
  // the db = 0 offset va gives block db at va ^ (64 db) (CPR 16) or va ^ (64 db)
  // with db < 2 (CPR 8: swz 4((r/2)%2) touches bit 2 of the chunk as well).
  const int vrow0 = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int vcol0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int va = tile_off<C::CPR, SWZ_TR>(vrow0, vcol0);
  auto kaddr = [&](int cc) __attribute__((always_inline)) { return ka ^ (32 * cc); };
  auto vaddr = [&](int db) __attribute__((always_inline)) { return va ^ (64 * db); };

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kMInit;    // running max, log2-scaled units (same in both lane halves)
  float lsum = 0.f;    // this lane's share of the running sum
  f32x16 s[NSB];       // scores of the tile between its matrix and softmax phases
  uint32_t pk[NSB][8]; // bf16 probabilities between the softmax and value phases

  // Matrix phase of round j: O^T += V^T P^T for tile j - 1 (skipped in the
  // first round) and the scores S^T = K Q^T of tile j (skipped in the last),
  // in steps of two value-product MFMAs (one 16-key chunk, two 32-feature
  // blocks) and two score MFMAs (16-feature k-step t of both 32-key
  // sub-blocks), issued value, score, value, score: the two score
  // accumulators are independent chains, so no MFMA waits on the one just
  // before it (one wave per SIMD issues every MFMA of a phase).  The operands of
  // step t + 1 are read from LDS (into the other half of a double buffer)
  // before the MFMAs of step t are issued, so the LDS latency hides behind
  // the matrix work; scheduling barriers keep that order.
  //
  // Every wave computes whole tiles, also on the causal diagonal where some
  // of its sub-blocks are masked entirely: the groups advance in lock step,
  // so a phase lasts as long as its busiest wave and skipping work in one
  // wave would not shorten it.  The softmax phase masks those scores.
  struct StepOps {
    bf16x8 v[2];   // V^T blocks
    bf16x8 k[2];   // K rows
  };
  enum { FIRST = 0, MID = 1, LAST = 2 };
  auto matrix_phase = [&](auto parity, auto kind) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;   // j & 1
    constexpr int KIND = decltype(kind)::value;
    constexpr bool DO_PV = KIND != FIRST;
    constexpr bool DO_S = KIND != LAST;
    constexpr int SUB = C::NDB / 2;              // steps per 16-key chunk
    constexpr int NSTEP = 2 * NSB * SUB;
    static_assert(C::NQC / 2 == 2 * SUB, "two score k-steps per step");
    const char* vs = smem_raw + C::OFF_V + (P ^ 1) * C::TILE_BYTES;
    const char* ks = smem_raw + P * C::TILE_BYTES;
    // step t: chunk kc = t / SUB (sub-block kc / 2, half kc % 2), part u = t % SUB
    auto load = [&](StepOps& o, int t) __attribute__((always_inline)) {
      const int kc = t / SUB, u = t % SUB, sb = kc >> 1, half = kc & 1;
      if constexpr (DO_PV) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int db = 2 * u + i;
          const u32x2 lo = lds_read_tr16(vs + vaddr(db) + (16 * kc) * C::ROW_BYTES);
          const u32x2 hi = lds_read_tr16(vs + vaddr(db) + (16 * kc + 8) * C::ROW_BYTES);
          o.v[i] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        }
      }
      if constexpr (DO_S) {
        // feature chunk t of both 32-key sub-blocks: two independent chains
#pragma unroll
        for (int i = 0; i < 2; ++i)
          o.k[i] = *reinterpret_cast<const bf16x8*>(ks + kaddr(t) + i * 32 * C::ROW_BYTES);
      }
    };
    auto compute = [&](const StepOps& o, int t) __attribute__((always_inline)) {
      const int kc = t / SUB, u = t % SUB, sb = kc >> 1, half = kc & 1;
      static_assert(NSTEP == C::NQC && NSB == 2, "one feature chunk per step");
      if constexpr (DO_S) {
        if (t == 0) {
          const f32x16 zero = {};
          s[0] = zero;
          s[1] = zero;
        }
      }
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, u32x4{pk[sb][4 * half + 0], pk[sb][4 * half + 1], pk[sb][4 * half + 2],
                        pk[sb][4 * half + 3]});
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (DO_PV) acc[2 * u + i] = mfma_32x32x16_bf16(o.v[i], b, acc[2 * u + i]);
        if constexpr (DO_S) s[i] = mfma_32x32x16_bf16(o.k[i], qf[t], s[i]);
      }
    };
    __builtin_amdgcn_s_setprio(1);
    StepOps ops[2];
    load(ops[0], 0);
#pragma unroll
    for (int t = 0; t < NSTEP; ++t) {
      if (t + 1 < NSTEP) load(ops[(t + 1) & 1], t + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(ops[t & 1], t);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // P = exp2(s*c - m), rounded to bf16 into pk; returns this lane's fp32 sum
  // of the unrounded p (the saved lse needs the unrounded sum: rounding each p
  // to bf16 first moves ln(l) by up to 2^-9 on short rows).
  auto probs = [&]() __attribute__((always_inline)) {
    float part[4];   // four partial sums: no serial add chain
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], c, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r + 1], c, -m));
        pk[sb][r >> 1] = pack_bf16x2(p0, p1);
        // the first pair of each partial sum starts it (no add of 0)
        if (sb == 0 && r < 8)
          part[(r >> 1) & 3] = p0 + p1;
        else
          part[(r >> 1) & 3] += p0 + p1;
      }
    return (part[0] + part[1]) + (part[2] + part[3]);
  };

  // Softmax phase of round j for tile j: mask, probabilities against the
  // current m; if some lane's sum passed the bound, move m to the true running
  // max (both halves of a query agree on it), rescale the accumulator and the
  // running sum by exp2(m_old - m_new) ("LLM Architecture Refresh [3]",
  // sections 2 and 4) and form the probabilities again.
  auto softmax_phase = [&](int j) __attribute__((always_inline)) {
    if (j < 0 || j >= nkt) return;
    const int k0 = kb + j * BN;
    if (CAUSAL && k0 > wq0 + 31 + koff) {
      // every key of the tile after every query of the wave: P = 0
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int i = 0; i < 8; ++i) pk[sb][i] = 0u;
      return;
    }
    if ((k0 + BN > ke) || (CAUSAL && k0 + BN - 1 > wq0 + koff)) {
      // register r of sub-block sb holds key k0 + 4h + off(sb, r) with
      // off = 32sb + 8(r/4) + r%4; it is dead past the lane's limit (the
      // last key its query sees under causal masking, and ke - 1).  Scores
      // of a tile with no visible key give p = 0: m is finite (kMInit or a
      // real maximum), so exp2(-inf - m) = 0 and no rebase is triggered.
      // Sub-blocks wholly visible to the wave keep their scores; wholly
      // invisible ones take -inf without a compare.
      int lim = ke - 1 - k0 - 4 * h;
      if (CAUSAL) lim = min(lim, qrow + koff - k0 - 4 * h);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int sk0 = k0 + 32 * sb;
        const bool full = sk0 + 31 < ke && (!CAUSAL || sk0 + 31 <= wq0 + koff);
        const bool dead = sk0 >= ke || (CAUSAL && sk0 > wq0 + 31 + koff);
        if (dead) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[sb][r] = kNegInf;
        } else if (!full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * sb + 8 * (r >> 2) + (r & 3);
            s[sb][r] = off > lim ? kNegInf : s[sb][r];
          }
        }
      }
    }
    float ps = probs();
    if (__any(ps > kSumBound)) {
      float mx = kNegInf;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      lsum *= alpha;
      m = m_new;
      ps = probs();
    }
    lsum += ps;
  };

  // Rounds j = 0 .. nkt.  Group 0: matrix phase j, softmax phase j; group 1:
  // softmax phase j - 1, matrix phase j.  At any time one wave of each SIMD
  // issues matrix-core work and the other vector work.  The tiles a round
  // reads were issued one round earlier and waited for at its end.
  // The two groups run separate loops (the same number of barriers): inside
  // one loop the scores are live across the back edge for one group and the
  // probabilities for the other, and merging the two would keep both live.
  // The DMAs go with the softmax phases: group 1 issues K tile j + 1 as round
  // j begins, group 0 V tile j as its softmax half begins.
  auto round = [&](int j, auto parity, auto group, auto kind) __attribute__((always_inline)) {
    constexpr int G = decltype(group)::value;
    if (G == 1 && j + 1 < nkt) issue(j + 1, 0u, Kb, koffA, koffB, rows_t{});
    if constexpr (G == 0) {
      matrix_phase(parity, kind);
      phase_barrier();
      if (j < nkt) issue(j, (unsigned)C::OFF_V, Vb, voffA, voffB, tr_t{});
      softmax_phase(j);
    } else {
      softmax_phase(j - 1);
      phase_barrier();
      matrix_phase(parity, kind);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's DMAs landed, its LDS reads done
    phase_barrier();
  };
  using even = std::integral_constant<int, 0>;
  using odd = std::integral_constant<int, 1>;
  using first = std::integral_constant<int, FIRST>;
  using mid = std::integral_constant<int, MID>;
  using last = std::integral_constant<int, LAST>;
  // rounds: 0 (scores only), 1 .. nkt-1, nkt (value product only)
  auto run = [&](auto group) __attribute__((always_inline)) {
    round(0, even{}, group, first{});
    int j = 1;
    for (; j + 1 < nkt; j += 2) {
      round(j, odd{}, group, mid{});
      round(j + 1, even{}, group, mid{});
    }
    if (j < nkt) {
      round(j, odd{}, group, mid{});
      ++j;
    }
    if (j & 1)
      round(j, odd{}, group, last{});
    else
      round(j, even{}, group, last{});
  };
  wait_vmem();
  phase_barrier();
  // Q^T as the B operand: lane holds Q[qrow][16c + 8h .. 16c + 8h + 7], at
  // row n of the wave's block in the query tile, chunk (2c + h) ^ (n % 16).
  {
    const uint32_t flip = a.negq ? 0x80008000u : 0u;
    const char* qs = smem_raw + C::OFF_Q + wblk * 32 * C::ROW_BYTES;
#pragma unroll
    for (int cc = 0; cc < C::NQC; ++cc) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qs + kaddr(cc));
      raw ^= flip;
      qf[cc] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  if (nkt > 0) {
    if (grp == 0)
      run(std::integral_constant<int, 0>{});
    else
      run(std::integral_constant<int, 1>{});
  }

  // epilogue: one deferred division, then O and the log-sum-exp.  A row
  // that saw no key (only possible with Nq > Nk, or in a key range wholly
  // after it) has l = 0: O = 0 and lse = -inf, the merge law's empty block.
  const float lt = lsum + wave_xor32(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  if (a.nsplit == 1) {
    // O goes through LDS (the K/V stages: every wave is past its last matrix
    // phase) so the stores are whole rows: the wave writes its 32 x D block
    // (row swizzle), then stores 16-byte chunks, 4 rows per instruction.
    char* ost = smem_raw + wblk * 32 * C::ROW_BYTES;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        u32x2 out = {pack_bf16x2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                     pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(ost + tile_off<C::CPR, SWZ_ROWS>(n, d0)) = out;
      }
    constexpr int PER = 64 / C::CPR;   // rows per store instruction
#pragma unroll
    for (int it = 0; it < 32 / PER; ++it) {
      const int r = it * PER + lane / C::CPR, ch = lane % C::CPR;
      const u32x4 v16 = *reinterpret_cast<const u32x4*>(ost + tile_off<C::CPR, SWZ_ROWS>(r, 8 * ch));
      if (wq0 + r < Nq)
        *reinterpret_cast<u32x4*>(a.O + base + (size_t)(wq0 + r) * D + 8 * ch) = v16;
    }
    if (h == 0 && qrow < Nq) a.LSE[(size_t)bh * Nq + qrow] = lse;
  } else if (qrow < Nq) {
    {
      const size_t prow = ((size_t)sp * BH + bh) * Nq + qrow;
      float* orow = a.Opart + prow * D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * h;
          f32x4 out = {acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                       acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + d0) = out;
        }
      if (h == 0) a.Lpart[prow] = lse;
    }
  }
}

// In-order forward for head dimension 64 ("Flash Attention, From First
// Principles", "The rent arithmetic": at d = 64 a score costs half the matrix
// work of d = 128 while its softmax costs the same, so the vector ALU, not the
// matrix core, sets the pace).  Measured on this chip: a wave64 v_fma_f32
// occupies a SIMD's vector ALU ~4 cycles and a v_exp_f32 ~8, so the softmax
// of a 32 x 64 tile (32 exponentials and ~80 other vector instructions per
// lane) costs about as much vector time as the tile's 16 matrix instructions
// cost matrix time, and one wave alone issues vector instructions well below
// the ALU's rate (an FMA every ~7 cycles).  The ping-pong kernel above lets
// only one wave per SIMD run softmax at a time; here every wave simply runs
//   S^T = K Q^T (MFMA) -> mask -> probabilities (lazy rebase) -> O^T += V^T P^T
// on its own 32 queries, a 64-key tile per round in two halves of 32 keys
// (half the score registers live at once: 4 workgroups fit a CU), and four
// workgroups of 4 waves x 32 queries share each CU, so at any time some waves
// of a SIMD keep its vector ALU busy while others feed its matrix core.  K and
// V tiles arrive by DMA, two stages deep, one barrier per round; the query
// tile arrives by DMA into the second stage (free until the first prefetch)
// and goes into registers from there.  A wave skips key tiles (and halves)
// wholly in the future of all its queries.
constexpr int kWavesIO = 4;
constexpr int kBMIO = 32 * kWavesIO;
constexpr int kBNIO = 64;
static_assert(kBMIO == fwd_rows_per_tile(64), "plan geometry");

template <int D>
struct IoCfg {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int ROW = CPR * 16;               // bytes per row
  static constexpr int TILE = kBNIO * ROW;           // one K or V tile
  static constexpr int STAGE = 2 * TILE;             // K then V
  static constexpr int NQC = D / 16;                 // k-steps of the score product
  static constexpr int NDB = D / 32;                 // 32-feature output blocks
  static constexpr int NSB = kBNIO / 32;             // 32-key sub-blocks
  static constexpr int DMA = TILE / (16 * 64 * kWavesIO);       // DMAs per lane per tile
  static constexpr int QDMA = kBMIO * ROW / (16 * 64 * kWavesIO);
  static constexpr int SMEM = 2 * STAGE;
  static_assert(kBMIO * ROW == STAGE, "the query tile fills the second stage");
  static_assert(DMA * 16 * 64 * kWavesIO == TILE, "DMA split");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 4) void fwd_inorder_kernel(const FwdArgs a) {
  using C = IoCfg<D>;
  constexpr int BN = kBNIO;
  constexpr int NSB = C::NSB;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  const int BH = a.BH, Nq = a.Nq, Nk = a.Nk, koff = a.koff;
  const float c = a.c;

  int bh, qt, sp = 0;
  {
    int bid = blockIdx.x;
    if (a.nsplit > 1) {
      sp = bid % a.nsplit;
      bid /= a.nsplit;
    }
    map_tile_snake(bid, BH, a.nqt, CAUSAL, a.pass, &bh, &qt);
  }
  const size_t base = (size_t)bh * (size_t)Nq * D;
  const size_t kvbase = (size_t)(bh / a.group) * (size_t)Nk * D;
  const char* Kb = reinterpret_cast<const char*>(a.K + kvbase);
  const char* Vb = reinterpret_cast<const char*>(a.V + kvbase);
  const int q0 = qt * kBMIO;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + n;

  const int kb = sp * a.klen;
  int ke = min(Nk, kb + a.klen);
  if (CAUSAL) ke = min(ke, q0 + kBMIO + koff);
  const int nkt = ke > kb ? (ke - kb + BN - 1) / BN : 0;

  // stage s holds K tile t (t & 1 == s) at s * STAGE and V tile t at
  // s * STAGE + TILE.  DMA slot (i * WAVES + w) * 64 + lane; rows past Nk are
  // clamped to row Nk - 1 (finite data; those keys are masked to -inf)
  const unsigned ldsb = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int k0 = kb + t * BN;
    const char* gk = Kb + (size_t)k0 * C::ROW;
    const char* gv = Vb + (size_t)k0 * C::ROW;
    const unsigned st = ldsb + (t & 1) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::DMA; ++i) {
      const int slot = (i * kWavesIO + w) * 64 + lane;
      const int row = slot / C::CPR;
      const int src_row = min(k0 + row, Nk - 1) - k0;
      const int ck = (slot % C::CPR) ^ swz<C::CPR, SWZ_ROWS>(row);
      const int cv = (slot % C::CPR) ^ swz<C::CPR, SWZ_TR>(row);
      const unsigned dst = (unsigned)((i * kWavesIO + w) * 1024);
      dma16(gk, (unsigned)(src_row * C::ROW + ck * 16), st + dst);
      dma16(gv, (unsigned)(src_row * C::ROW + cv * 16), st + C::TILE + dst);
    }
  };
  if (nkt > 0) issue(0);

  // the query tile by whole-row DMA into stage 1 (row swizzle; rows past Nq
  // fall outside the buffer resource and read 0).  Wave w fills slots w,
  // w + 4, ..; DMA i + 1 is DMA i shifted by 4 KiB on both sides (a multiple
  // of the swizzle's 16-row period).
  {
    static_assert((kWavesIO * 1024 / C::ROW) % 16 == 0, "swizzle period");
    const int slot = w * 64 + lane;
    const int row = slot / C::CPR;
    const int chunk = (slot % C::CPR) ^ swz<C::CPR, SWZ_ROWS>(row);
    const unsigned qoff = (unsigned)((row * D + chunk * 8) * 2);
    const long long qbytes = (long long)max(0, Nq - q0) * (D * 2);
    const char* Qt = reinterpret_cast<const char*>(a.Q + base + (size_t)q0 * D);
#pragma unroll
    for (int i = 0; i < C::QDMA; ++i) {
      const long long b0 = (long long)i * 1024 * kWavesIO;
      const long long nrec = qbytes - b0 > 0 ? qbytes - b0 : 0;
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(Qt + b0), (short)0, (int)nrec, 0x00020000);
      dma16_buf(rsrc, qoff, ldsb + C::STAGE + (unsigned)b0 + w * 1024);
    }
  }
  // K operand (A of S^T): row 32 sb + n, features 16 cc + 8 h; V^T operand
  // through transposing reads (the ping-pong kernel's patterns)
  const int ka = tile_off<C::CPR, SWZ_ROWS>(n, 8 * h);
  const int vrow0 = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int vcol0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int va = tile_off<C::CPR, SWZ_TR>(vrow0, vcol0);

  wait_vmem();
  __syncthreads();
  bf16x8 qf[C::NQC];
  {
    const uint32_t flip = a.negq ? 0x80008000u : 0u;
    const char* qs = smem_raw + C::STAGE + 32 * w * C::ROW;
#pragma unroll
    for (int cc = 0; cc < C::NQC; ++cc) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qs + (ka ^ (32 * cc)));
      raw ^= flip;
      qf[cc] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kMInit;
  float lsum = 0.f;
  bool fresh = true;   // no half processed yet (wave-uniform)

  for (int j = 0; j < nkt; ++j) {
    // tile j landed for every wave; every wave is done with tile j - 1 (and,
    // at j = 0, with the query tile in stage 1)
    wait_vmem();
    __syncthreads();
    if (j + 1 < nkt) issue(j + 1);
    // issue priority by remaining work: workgroups that have more rounds
    // left go first (the issue arbiter otherwise favours the oldest waves,
    // which then finish long before the rest and leave the SIMDs half idle)
    {
      const int rem = nkt - j;
      if (rem > a.prio3) __builtin_amdgcn_s_setprio(3);
      else if (rem > a.prio2) __builtin_amdgcn_s_setprio(2);
      else if (rem > a.prio1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    const int k0 = kb + j * BN;
    if (CAUSAL && k0 > wq0 + 31 + koff) continue;   // every key after every query
    const char* ks = smem_raw + (j & 1) * C::STAGE;
    const char* vs = ks + C::TILE;

    // the tile in two halves of 32 keys (half the score and probability
    // registers of a whole tile live at once): per half S^T (lane = query;
    // register r holds key k0 + 32 sb + 8 (r / 4) + 4 h + r % 4), mask,
    // probabilities against the running max (lazy rebase), O^T += V^T P^T
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      if (CAUSAL && k0 + 32 * sb > wq0 + 31 + koff) break;   // the rest is all future
      f32x16 s = {};
#pragma unroll
      for (int cc = 0; cc < C::NQC; ++cc) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(ks + (ka ^ (32 * cc)) + sb * 32 * C::ROW);
        s = mfma_32x32x16_bf16(kf, qf[cc], s);
      }
      // a half wholly visible to the wave (keys before every query, all < ke)
      // needs no mask
      if ((k0 + 32 * sb + 32 > ke) || (CAUSAL && k0 + 32 * sb + 31 > wq0 + koff)) {
        int lim = ke - 1 - k0 - 32 * sb - 4 * h;
        if (CAUSAL) lim = min(lim, qrow + koff - k0 - 32 * sb - 4 * h);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          s[r] = off > lim ? kNegInf : s[r];
        }
      }
      uint32_t pk[8];
      auto probs = [&]() __attribute__((always_inline)) {
        float part[4];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], c, -m));
          pk[r >> 1] = pack_bf16x2(p0, p1);
          if (r < 8)
            part[(r >> 1) & 3] = p0 + p1;
          else
            part[(r >> 1) & 3] += p0 + p1;
        }
        return (part[0] + part[1]) + (part[2] + part[3]);
      };
      if (fresh) {
        // the wave's first half: m takes the true running max before any
        // probability (against m's start value every p would overflow and
        // force the rebase below); acc and l are still zero
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, wave_xor32(mx));
        m = fmaxf(m, mx * c);
        fresh = false;
      }
      float ps = probs();
      if (__any(ps > kSumBound)) {
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, wave_xor32(mx));
        const float m_new = fmaxf(m, mx * c);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        lsum *= alpha;
        m = m_new;
        ps = probs();
      }
      lsum += ps;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 b = __builtin_bit_cast(
            bf16x8, u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]});
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const char* vp = vs + (va ^ (64 * db)) + (32 * sb + 16 * half) * C::ROW;
          const u32x2 lo = lds_read_tr16(vp);
          const u32x2 hi = lds_read_tr16(vp + 8 * C::ROW);
          acc[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}),
                                       b, acc[db]);
        }
      }
    }
  }

  // epilogue: one deferred division, then O and the log-sum-exp.  A row that
  // saw no key has l = 0: O = 0 and lse = -inf, the merge law's empty block.
  const float lt = lsum + wave_xor32(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  if (a.nsplit == 1) {
    // O through LDS (stage 0, after every wave's last read) as whole rows:
    // the wave writes its 32 x D block (row swizzle), then stores 16-byte
    // chunks, 64 / CPR rows per instruction
    __syncthreads();
    char* ost = smem_raw + 32 * w * C::ROW;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        u32x2 out = {pack_bf16x2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                     pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(ost + tile_off<C::CPR, SWZ_ROWS>(n, d0)) = out;
      }
    constexpr int PER = 64 / C::CPR;
#pragma unroll
    for (int it = 0; it < 32 / PER; ++it) {
      const int r = it * PER + lane / C::CPR, ch = lane % C::CPR;
      const u32x4 v16 =
          *reinterpret_cast<const u32x4*>(ost + tile_off<C::CPR, SWZ_ROWS>(r, 8 * ch));
      if (wq0 + r < Nq)
        *reinterpret_cast<u32x4*>(a.O + base + (size_t)(wq0 + r) * D + 8 * ch) = v16;
    }
    if (h == 0 && qrow < Nq) a.LSE[(size_t)bh * Nq + qrow] = lse;
  } else if (qrow < Nq) {
    const size_t prow = ((size_t)sp * BH + bh) * Nq + qrow;
    float* orow = a.Opart + prow * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        f32x4 out = {acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                     acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + d0) = out;
      }
    if (h == 0) a.Lpart[prow] = lse;
  }
}

// Head dimension 256 ("Flash Attention, From First Principles", "The rent
// arithmetic": the accumulator and the query tile grow with d, the tiles
// shrink).  The ping-pong kernel above needs ~270 registers per wave at this
// size, so this kernel has no second group: per 32-key tile a wave forms
// S^T = K Q^T (16 MFMAs), the probabilities against its running max (same
// lazy rebase as above), and O^T += V^T P^T (16 MFMAs), in order.  Two
// workgroups share a CU (two waves per SIMD, 256 registers each: the 32 x 256
// accumulator 128, the query operands 64, the rest the scores, probabilities
// and operand reads), so one workgroup's vector work overlaps the other's
// matrix work.  The per-lane DMA and operand offsets are formed where they
// are used (their bases opaque to the compiler): held for the whole loop they
// spilled, and the DMA addresses then came from scratch memory on the
// prefetch's path (1 workgroup per CU: 0.211 ms, 2 with the spills: 0.327 ms,
// 2 without: 0.181 ms at [1, 16, 4096, 256] causal).  K and V tiles arrive by
// DMA, two stages deep, one barrier per tile.  Workgroup: 4 waves x 32
// queries = 128 queries, 64 KiB of LDS.
constexpr int kWaves256 = 4;
constexpr int kBM256 = 32 * kWaves256;
static_assert(kBM256 == fwd_rows_per_tile(256), "plan geometry");
constexpr int kBN256 = 32;

template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_d256_kernel(const FwdArgs a) {
  constexpr int D = 256;
  constexpr int BN = kBN256;
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int ROW = CPR * 16;               // bytes per row
  constexpr int TILE = BN * ROW;              // one K or V tile (16 KiB)
  constexpr int NQC = D / 16;                 // k-steps of the score product
  constexpr int NDB = D / 32;                 // 32-feature output blocks
  constexpr int DMA = TILE / (16 * 64 * kWaves256);   // DMAs per lane per tile
  constexpr int OFF_V = 2 * TILE;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  const int BH = a.BH, Nq = a.Nq, Nk = a.Nk, koff = a.koff;
  const float c = a.c;

  int bh, qt, sp = 0;
  {
    int bid = blockIdx.x;
    if (a.nsplit > 1) {
      sp = bid % a.nsplit;
      bid /= a.nsplit;
    }
    map_tile_snake(bid, BH, a.nqt, CAUSAL, a.pass, &bh, &qt);
  }
  const size_t base = (size_t)bh * (size_t)Nq * D;
  const size_t kvbase = (size_t)(bh / a.group) * (size_t)Nk * D;
  const char* Kb = reinterpret_cast<const char*>(a.K + kvbase);
  const char* Vb = reinterpret_cast<const char*>(a.V + kvbase);
  const int q0 = qt * kBM256;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + n;

  const int kb = sp * a.klen;
  int ke = min(Nk, kb + a.klen);
  if (CAUSAL) ke = min(ke, q0 + kBM256 + koff);
  const int nkt = ke > kb ? (ke - kb + BN - 1) / BN : 0;

  // DMA of tile t into stage t & 1: slot (i * 4 + w) * 64 + lane of the tile
  const unsigned ldsb = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int k0 = kb + t * BN;
    const char* gk = Kb + (size_t)k0 * ROW;
    const char* gv = Vb + (size_t)k0 * ROW;
    const unsigned stk = ldsb + (t & 1) * TILE;
    const unsigned stv = ldsb + OFF_V + (t & 1) * TILE;
    const int ln = opaque(lane);
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const int slot = (i * kWaves256 + w) * 64 + ln;
      const int row = slot / CPR;
      const int src_row = min(k0 + row, Nk - 1) - k0;
      const int ck = (slot % CPR) ^ swz<CPR, SWZ_ROWS>(row);
      const int cv = (slot % CPR) ^ swz<CPR, SWZ_TR>(row);
      const unsigned dst = (unsigned)((i * kWaves256 + w) * 1024);
      dma16(gk, (unsigned)(src_row * ROW + ck * 16), stk + dst);
      dma16(gv, (unsigned)(src_row * ROW + cv * 16), stv + dst);
    }
  };
  if (nkt > 0) issue(0);

  bf16x8 qf[NQC];
  {
    const uint32_t flip = a.negq ? 0x80008000u : 0u;
    const uint16_t* Qh = a.Q + base;
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qrow < Nq)
        raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + 16 * cc + 8 * h);
      raw ^= flip;
      qf[cc] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const int ka = tile_off<CPR, SWZ_ROWS>(n, 8 * h);
  const int vrow0 = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int vcol0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int va = tile_off<CPR, SWZ_TR>(vrow0, vcol0);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kMInit;
  float lsum = 0.f;

  for (int j = 0; j < nkt; ++j) {
    // tile j landed for every wave; every wave is done with tile j - 1
    wait_vmem();
    __syncthreads();
    if (j + 1 < nkt) issue(j + 1);
    const char* ks = smem_raw + (j & 1) * TILE;
    const char* vs = smem_raw + OFF_V + (j & 1) * TILE;
    const int k0 = kb + j * BN;
    if (CAUSAL && k0 > wq0 + 31 + koff) continue;   // every key after every query

    f32x16 s = {};
    const int ka_ = opaque(ka), va_ = opaque(va);
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (ka_ ^ (32 * cc)));
      s = mfma_32x32x16_bf16(kf, qf[cc], s);
    }
    if ((k0 + BN > ke) || (CAUSAL && k0 + BN - 1 > wq0 + koff)) {
      int lim = ke - 1 - k0 - 4 * h;
      if (CAUSAL) lim = min(lim, qrow + koff - k0 - 4 * h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        s[r] = off > lim ? kNegInf : s[r];
      }
    }
    uint32_t pk[8];
    auto probs = [&]() __attribute__((always_inline)) {
      float part[2] = {0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], c, -m));
        pk[r >> 1] = pack_bf16x2(p0, p1);
        part[(r >> 1) & 1] += p0 + p1;
      }
      return part[0] + part[1];
    };
    float ps = probs();
    if (__any(ps > kSumBound)) {
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      lsum *= alpha;
      m = m_new;
      ps = probs();
    }
    lsum += ps;

#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]});
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* vp = vs + (va_ ^ (64 * db)) + 16 * half * ROW;
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 8 * ROW);
        acc[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}),
                                     b, acc[db]);
      }
    }
  }

  const float lt = lsum + wave_xor32(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  if (qrow < Nq) {
    if (a.nsplit == 1) {
      uint16_t* orow = a.O + base + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * h;
          u32x2 out = {pack_bf16x2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                       pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = out;
        }
      if (h == 0) a.LSE[(size_t)bh * Nq + qrow] = lse;
    } else {
      const size_t prow = ((size_t)sp * BH + bh) * Nq + qrow;
      float* orow = a.Opart + prow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * h;
          f32x4 out = {acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                       acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + d0) = out;
        }
      if (h == 0) a.Lpart[prow] = lse;
    }
  }
}

// Causal head dimension 256 with balanced workgroups.  Two workgroups of the
// kernel above share a CU, and under causal masking with exactly one
// workgroup per slot (B*H*N/128 = 2 x CUs) the CU that holds a short and a
// long tile runs the long one alone, at one wave per SIMD, for most of the
// kernel ([1, 16, 4096, 256]: 31 % of peak causal against 43 % non-causal).
// Here one workgroup of two groups of four waves (two waves per SIMD, the
// same register budget) owns the pair of query tiles p and nqt - 1 - p of one
// head, whose causal key ranges add up to the same length for every p, and
// deals the key tiles so both groups do the same number of rounds: group 1
// takes the first s key tiles of the heavy tile, group 0 the whole light tile
// and then the heavy tile's remaining key tiles.  Each group streams its own
// K / V tiles through its own two LDS stages; one workgroup barrier per
// round.  At the end the heavy tile's two partial results -- (running max,
// running sum, unnormalised output) of the same rows over disjoint key ranges
// -- are merged through LDS by the composite-block law of "Flash Attention,
// From First Principles", "The scaffold" (rescale both by exp(m_part - m),
// add), and group 0 writes the output.
template <bool CAUSAL>
__global__ __launch_bounds__(512, 2) void fwd_d256_pair_kernel(const FwdArgs a) {
  constexpr int D = 256;
  constexpr int BN = kBN256;
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int ROW = CPR * 16;               // bytes per row
  constexpr int TILE = BN * ROW;              // one K or V tile (16 KiB)
  constexpr int NQC = D / 16;                 // k-steps of the score product
  constexpr int NDB = D / 32;                 // 32-feature output blocks
  constexpr int DMA = TILE / (16 * 64 * kWaves256);   // DMAs per lane per tile
  constexpr int OFF_V = 2 * TILE;
  constexpr int GROUP_LDS = 4 * TILE;         // a group's two K / V stages
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wg >> 2;                    // wave wg runs on SIMD wg % 4
  const int w = wg & 3;                       // 32-query block inside a tile
  const int n = lane & 31;
  const int h = lane >> 5;
  const int BH = a.BH, Nq = a.Nq, Nk = a.Nk, koff = a.koff;
  const float c = a.c;

  // pair p of head bh; whole heads per XCD when the head count allows
  int bh, p;
  {
    const int bid = blockIdx.x;
    if ((BH & 7) == 0) {
      const int j = bid >> 3, hpx = BH >> 3;
      p = j / hpx;
      bh = (bid & 7) * hpx + (j - p * hpx);
    } else {
      p = bid / BH;
      bh = bid - p * BH;
    }
  }
  const int ta = p, tb = a.nqt - 1 - p;       // light and heavy tile
  auto nkt_of = [&](int qt) {
    const int ke = min(Nk, qt * kBM256 + kBM256 + koff);
    return ke > 0 ? (ke + BN - 1) / BN : 0;
  };
  const int ra = nkt_of(ta), rb = nkt_of(tb);
  const int sk = (ra + rb + 1) / 2;           // group 1: heavy tile's key tiles [0, sk)
  const int nr = grp ? sk : ra + rb - sk;     // this group's rounds (group 0's <= group 1's)

  const size_t kvbase = (size_t)(bh / a.group) * (size_t)Nk * D;
  const char* Kb = reinterpret_cast<const char*>(a.K + kvbase);
  const char* Vb = reinterpret_cast<const char*>(a.V + kvbase);
  const size_t base = (size_t)bh * (size_t)Nq * D;

  // round j of this group -> key tile index of its current query tile
  auto key_tile = [&](int j) { return grp ? j : (j < ra ? j : sk + (j - ra)); };

  // DMA of round t into this group's stage t & 1
  const unsigned ldsb = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw)) + grp * GROUP_LDS;
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int k0 = key_tile(t) * BN;
    const char* gk = Kb + (size_t)k0 * ROW;
    const char* gv = Vb + (size_t)k0 * ROW;
    const unsigned stk = ldsb + (t & 1) * TILE;
    const unsigned stv = ldsb + OFF_V + (t & 1) * TILE;
    const int ln = opaque(lane);
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const int slot = (i * kWaves256 + w) * 64 + ln;
      const int row = slot / CPR;
      const int src_row = min(k0 + row, Nk - 1) - k0;
      const int ck = (slot % CPR) ^ swz<CPR, SWZ_ROWS>(row);
      const int cv = (slot % CPR) ^ swz<CPR, SWZ_TR>(row);
      const unsigned dst = (unsigned)((i * kWaves256 + w) * 1024);
      dma16(gk, (unsigned)(src_row * ROW + ck * 16), stk + dst);
      dma16(gv, (unsigned)(src_row * ROW + cv * 16), stv + dst);
    }
  };
  if (nr > 0) issue(0);

  // the group's current query tile: group 1 the heavy one, group 0 the light
  // one and, from round ra on, the heavy one
  int qt = grp ? tb : ta;
  int wq0 = qt * kBM256 + 32 * w;
  int qrow = wq0 + n;
  int ke = min(Nk, qt * kBM256 + kBM256 + koff);
  bf16x8 qf[NQC];
  auto load_q = [&]() __attribute__((always_inline)) {
    const uint32_t flip = a.negq ? 0x80008000u : 0u;
    const uint16_t* Qh = a.Q + base;
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qrow < Nq)
        raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + 16 * cc + 8 * h);
      raw ^= flip;
      qf[cc] = __builtin_bit_cast(bf16x8, raw);
    }
  };
  load_q();
  const int ka = tile_off<CPR, SWZ_ROWS>(n, 8 * h);
  const int vrow0 = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int vcol0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int va = tile_off<CPR, SWZ_TR>(vrow0, vcol0);

  f32x16 acc[NDB];
  float m, lsum;
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    m = kMInit;
    lsum = 0.f;
  };
  reset();
  // one deferred division, then O and the log-sum-exp of the current tile
  auto store_out = [&]() __attribute__((always_inline)) {
    const float lt = lsum + wave_xor32(lsum);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
    if (qrow < Nq) {
      uint16_t* orow = a.O + base + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * h;
          u32x2 out = {pack_bf16x2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                       pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = out;
        }
      if (h == 0) a.LSE[(size_t)bh * Nq + qrow] = lse;
    }
  };
  // group 0: the light tile is done -- its output out, the heavy tile's rows in
  auto switch_tile = [&]() __attribute__((always_inline)) {
    store_out();
    qt = tb;
    wq0 = qt * kBM256 + 32 * w;
    qrow = wq0 + n;
    ke = min(Nk, qt * kBM256 + kBM256 + koff);
    load_q();
    reset();
  };

  for (int j = 0; j < sk; ++j) {
    // this group's tile j landed for its waves; every wave is done with round j - 1
    wait_vmem();
    __syncthreads();
    if (j >= nr) continue;                    // group 0 with one round fewer
    if (j + 1 < nr) issue(j + 1);
    if (grp == 0 && j == ra) switch_tile();
    const char* ks = smem_raw + grp * GROUP_LDS + (j & 1) * TILE;
    const char* vs = smem_raw + grp * GROUP_LDS + OFF_V + (j & 1) * TILE;
    const int k0 = key_tile(j) * BN;
    if (CAUSAL && k0 > wq0 + 31 + koff) continue;   // every key after every query

    f32x16 s = {};
    const int ka_ = opaque(ka), va_ = opaque(va);
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (ka_ ^ (32 * cc)));
      s = mfma_32x32x16_bf16(kf, qf[cc], s);
    }
    if ((k0 + BN > ke) || (CAUSAL && k0 + BN - 1 > wq0 + koff)) {
      int lim = ke - 1 - k0 - 4 * h;
      if (CAUSAL) lim = min(lim, qrow + koff - k0 - 4 * h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        s[r] = off > lim ? kNegInf : s[r];
      }
    }
    uint32_t pk[8];
    auto probs = [&]() __attribute__((always_inline)) {
      float part[2] = {0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], c, -m));
        pk[r >> 1] = pack_bf16x2(p0, p1);
        part[(r >> 1) & 1] += p0 + p1;
      }
      return part[0] + part[1];
    };
    float ps = probs();
    if (__any(ps > kSumBound)) {
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      lsum *= alpha;
      m = m_new;
      ps = probs();
    }
    lsum += ps;

#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]});
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* vp = vs + (va_ ^ (64 * db)) + 16 * half * ROW;
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 8 * ROW);
        acc[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}),
                                     b, acc[db]);
      }
    }
  }
  // group 0 took no key tile of the heavy tile: the light tile is still open
  // and the heavy tile's share of group 0 is empty (m = kMInit, sum 0)
  if (grp == 0 && nr == ra) switch_tile();

  // merge the heavy tile: group 1 parks (acc, m, sum) in LDS (the stages are
  // free: every wave is past its last round), group 0 adds it to its own
  // share with both rescaled to the larger max, and writes the rows
  __syncthreads();
  char* park = smem_raw + w * (NDB * 16 * 64 * 4);   // 32 KiB per 32-row block
  float* park_ml = reinterpret_cast<float*>(smem_raw + 4 * NDB * 16 * 64 * 4) + 2 * (w * 64 + lane);
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(park + ((db * 4 + g) * 64 + lane) * 16) =
            f32x4{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
    park_ml[0] = m;
    park_ml[1] = lsum;
  }
  __syncthreads();
  if (grp == 0) {
    const float m1 = park_ml[0], l1 = park_ml[1];
    const float mm = fmaxf(m, m1);
    const float a0 = __builtin_amdgcn_exp2f(m - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(park + ((db * 4 + g) * 64 + lane) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * g + e] = acc[db][4 * g + e] * a0 + o1[e] * a1;
      }
    lsum = lsum * a0 + l1 * a1;
    m = mm;
    store_out();
  }
}

// FP8 forward ("LLM Architecture Refresh [3]", section 8: the FA-3 direction
// of lower-precision matrix inputs).  Q, K and V arrive as OCP e4m3 bytes
// with one dequantisation factor per tensor; both products run on
// v_mfma_f32_32x32x64_f8f6f4 (fp8 inputs, fp32 accumulation), so the
// probabilities are rounded to e4m3 for the P V product -- the error budget
// of this path (3 mantissa bits on each p) is stated with its tests.  The
// running max / sum, the rescale and the lse stay fp32 exactly as in the bf16
// kernels.  Head dimension 128; 4 waves x 32 queries per workgroup, 64-key
// tiles, one wave per SIMD (the fp8 products are half as long as the bf16
// ones, so a wave interleaves little and the structure is the d = 256 one).
//
// Operand layouts of the 32x32x64 fp8 MFMA (same lane / byte -> k mapping in
// A and B): lane l holds row (A) or column (B) l % 32 and 32 bytes, the k
// values of half l / 32.
//   S^T = K Q^T: A = K rows (32 consecutive features of the key per lane),
//       B = Q^T (the same 32 features of the query).
//   O^T += V^T P^T: B = P^T: lane (query n, half h) byte 16 sb + r holds p
//       of key 32 sb + 8 (r / 4) + 4 h + r % 4 (the S^T accumulator's own
//       registers, converted in place); A = V^T: four ds_read_b64_tr_b8 per
//       32-feature block, read t giving bytes 8 t .. 8 t + 7 = keys
//       16 t + 4 h + {0, 1, 2, 3, 8, 9, 10, 11} of that feature.
// ds_read_b64_tr_b8: in each 16-lane group, lane 2j + c reads 8 bytes of row
// j (bytes 8c .. 8c + 7 of a 16-byte column chunk); output lane i receives
// byte i of rows 0..7.  K tiles use the row swizzle (r / 2) % 8 on their
// 16-byte chunks (conflict-free for the row reads), V tiles swzv8 below
// (conflict-free for the transposing reads).
constexpr int kWavesF8 = 4;
constexpr int kBMF8 = 32 * kWavesF8;
constexpr int kBNF8 = 64;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ f32x16 mfma_32x32x64_f8(const i32x8& a, const i32x8& b,
                                                   const f32x16& c) {
  // formats 0 / 0: both operands e4m3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
// V tiles: ds_read_b64_tr_b8 reads, per 32 lanes, rows {0..3, 8..11} + c
// (c a multiple of 4), four lanes (two 8-byte halves of two 16-byte chunks)
// per row; 2 ((r / 2) % 2) + 4 ((r / 8) % 2) gives each of the four even and
// four odd rows its own chunk pair, so the 32 reads fill 32 distinct 8-byte
// bank slots (the row swizzle above maps rows r and r + 2 onto one pair)
__device__ __forceinline__ int swzv8(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }

// Two waves per SIMD (two workgroups per CU, each with its own barriers): the
// kernel issues a tile's matrix and vector work in order, and the other
// workgroup's wave fills the matrix core or the vector ALU meanwhile
// (N = 4096, d = 128 causal: 741 -> 1248 TFLOP/s against one wave per SIMD).
template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(const FwdArgs a, float vscale) {
  constexpr int D = 128;
  constexpr int BN = kBNF8;
  constexpr int ROW = D;                      // bytes per fp8 row
  constexpr int TILE = BN * ROW;              // 8 KiB
  constexpr int DMA = TILE / (16 * 64 * kWavesF8);   // DMAs per lane per tile
  constexpr int OFF_V = 2 * TILE;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  const int BH = a.BH, Nq = a.Nq, Nk = a.Nk, koff = a.koff;
  const float c = a.c;
  const unsigned char* Q8 = reinterpret_cast<const unsigned char*>(a.Q);
  const unsigned char* K8 = reinterpret_cast<const unsigned char*>(a.K);
  const unsigned char* V8 = reinterpret_cast<const unsigned char*>(a.V);

  int bh, qt, sp = 0;
  {
    int bid = blockIdx.x;
    if (a.nsplit > 1) {
      sp = bid % a.nsplit;
      bid /= a.nsplit;
    }
    map_tile_snake(bid, BH, a.nqt, CAUSAL, a.pass, &bh, &qt);
  }
  const size_t base = (size_t)bh * (size_t)Nq * D;
  const size_t kvbase = (size_t)(bh / a.group) * (size_t)Nk * D;
  const char* Kb = reinterpret_cast<const char*>(K8 + kvbase);
  const char* Vb = reinterpret_cast<const char*>(V8 + kvbase);
  const int q0 = qt * kBMF8;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + n;

  const int kb = sp * a.klen;
  int ke = min(Nk, kb + a.klen);
  if (CAUSAL) ke = min(ke, q0 + kBMF8 + koff);
  const int nkt = ke > kb ? (ke - kb + BN - 1) / BN : 0;

  const unsigned ldsb = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int k0 = kb + t * BN;
    const char* gk = Kb + (size_t)k0 * ROW;
    const char* gv = Vb + (size_t)k0 * ROW;
    const unsigned stk = ldsb + (t & 1) * TILE;
    const unsigned stv = ldsb + OFF_V + (t & 1) * TILE;
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const int slot = (i * kWavesF8 + w) * 64 + lane;
      const int row = slot / 8;
      const int src_row = min(k0 + row, Nk - 1) - k0;
      const unsigned srck = (unsigned)(src_row * ROW + ((slot % 8) ^ swz8(row)) * 16);
      const unsigned srcv = (unsigned)(src_row * ROW + ((slot % 8) ^ swzv8(row)) * 16);
      const unsigned dst = (unsigned)((i * kWavesF8 + w) * 1024);
      dma16(gk, srck, stk + dst);
      dma16(gv, srcv, stv + dst);
    }
  };
  if (nkt > 0) issue(0);

  // Q^T operand, k-steps cc = 0, 1: features 64 cc + 32 h .. + 31 (a
  // negative score factor flips the e4m3 sign bits: exact)
  i32x8 qf[2];
  const uint32_t flip = a.negq ? 0x80808080u : 0u;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (qrow < Nq) {
      const u32x4* src =
          reinterpret_cast<const u32x4*>(Q8 + base + (size_t)qrow * D + 64 * cc + 32 * h);
      lo = src[0] ^ flip;
      hi = src[1] ^ flip;
    }
    qf[cc] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  // K operand address of (sub-block sb, k-step cc, 16-byte part u): row
  // 32 sb + n, chunk 4 cc + 2 h + u
  auto koff_of = [&](int sb, int cc, int u) __attribute__((always_inline)) {
    const int row = 32 * sb + n;
    return row * ROW + (((4 * cc + 2 * h + u) ^ swz8(row)) << 4);
  };
  // V^T operand address of (feature block db, read t): row 16 t + 4 h +
  // 8 (j / 4) + j % 4, bytes 8 c of chunk 2 db + (lane % 32) / 16
  const int jv = (lane & 15) >> 1;
  const int cv = lane & 1;
  const int gv = (lane >> 4) & 1;
  // The swizzle sees row bits 1 and 3 only, so read t + 1 is read t moved
  // 16 rows down (an immediate offset): one base register per block db.
  auto voff_of = [&](int db, int t) __attribute__((always_inline)) {
    const int row = 16 * t + 4 * h + 8 * (jv >> 2) + (jv & 3);
    return row * ROW + (((2 * db + gv) ^ swzv8(row)) << 4) + 8 * cv;
  };
  int vbase[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) vbase[db] = voff_of(db, 0);

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kMInit;
  float lsum = 0.f;
  int pw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  bool fresh = true;   // no tile processed yet (wave-uniform)

  for (int j = 0; j < nkt; ++j) {
    wait_vmem();
    __syncthreads();
    if (j + 1 < nkt) issue(j + 1);
    const char* ks = smem_raw + (j & 1) * TILE;
    const char* vs = smem_raw + OFF_V + (j & 1) * TILE;
    const int k0 = kb + j * BN;
    if (CAUSAL && k0 > wq0 + 31 + koff) continue;   // every key after every query

    f32x16 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(ks + koff_of(sb, cc, 0));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(ks + koff_of(sb, cc, 1));
        const i32x8 kf = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        s[sb] = mfma_32x32x64_f8(kf, qf[cc], s[sb]);
      }
    }
    if ((k0 + BN > ke) || (CAUSAL && k0 + BN - 1 > wq0 + koff)) {
      // sub-blocks wholly visible to the wave keep their scores, wholly
      // invisible ones take -inf without a compare
      int lim = ke - 1 - k0 - 4 * h;
      if (CAUSAL) lim = min(lim, qrow + koff - k0 - 4 * h);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int sk0 = k0 + 32 * sb;
        const bool full = sk0 + 31 < ke && (!CAUSAL || sk0 + 31 <= wq0 + koff);
        const bool dead = sk0 >= ke || (CAUSAL && sk0 > wq0 + 31 + koff);
        if (dead) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[sb][r] = kNegInf;
        } else if (!full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * sb + 8 * (r >> 2) + (r & 3);
            s[sb][r] = off > lim ? kNegInf : s[sb][r];
          }
        }
      }
    }
    auto probs = [&]() __attribute__((always_inline)) {
      float part[4];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], c, -m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r + 1], c, -m));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r + 2], c, -m));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r + 3], c, -m));
          // the two conversions write the word's low and high halves: the
          // old contents (last tile's bytes) never survive, so no zeroing
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pw[4 * sb + (r >> 2)], false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
          pw[4 * sb + (r >> 2)] = word;
          // the first pair of each partial sum starts it (no add of 0)
          if (sb == 0)
            part[r >> 2] = (p0 + p1) + (p2 + p3);
          else
            part[r >> 2] += (p0 + p1) + (p2 + p3);
        }
      return (part[0] + part[1]) + (part[2] + part[3]);
    };
    if (fresh) {
      // the wave's first tile: m takes the true running max before any
      // probability (acc and l are still zero)
      float mx = kNegInf;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
      mx = fmaxf(mx, wave_xor32(mx));
      m = fmaxf(m, mx * c);
      fresh = false;
    }
    float ps = probs();
    if (__any(ps > kSumBound)) {
      float mx = kNegInf;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      lsum *= alpha;
      m = m_new;
      ps = probs();
    }
    lsum += ps;
    const i32x8 pb = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i32x2 r4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        r4[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2*)(vs + vbase[db] + 16 * t * ROW));
      const i32x8 vf = {r4[0].x, r4[0].y, r4[1].x, r4[1].y, r4[2].x, r4[2].y, r4[3].x, r4[3].y};
      acc[db] = mfma_32x32x64_f8(vf, pb, acc[db]);
    }
  }

  const float lt = lsum + wave_xor32(lsum);
  const float inv = lt > 0.f ? vscale / lt : 0.f;
  const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  if (qrow < Nq) {
    if (a.nsplit == 1) {
      uint16_t* orow = a.O + base + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * h;
          u32x2 out = {pack_bf16x2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                       pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = out;
        }
      if (h == 0) a.LSE[(size_t)bh * Nq + qrow] = lse;
    } else {
      const size_t prow = ((size_t)sp * BH + bh) * Nq + qrow;
      float* orow = a.Opart + prow * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * h;
          f32x4 out = {acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                       acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + d0) = out;
        }
      if (h == 0) a.Lpart[prow] = lse;
    }
  }
}

// Decode (few query rows per key / value head: generated tokens against a
// cache, "LLM Architecture Refresh [3]", section 6 and the notes on prompt and
// generated tokens).  The 256-query tile would compute 256 rows for each key
// tile and use a handful.  Here one wave owns EVERY query row that reads a key
// / value head -- the group's query heads times the Nq positions, R <= 32 rows
// packed into the 32 MFMA columns -- so each key and value byte is read once
// per key / value head, and each workgroup (one wave) streams one range of the
// keys.  S^T = K Q^T (lane = packed row), the lazy-rebase softmax and
// O^T += V^T P^T are the forward kernel's; ranges merge through
// fwd_merge_kernel.  32-key tiles by DMA, three stages (a wave's own, no
// barrier): tile j is read while tiles j + 1 and j + 2 are in flight.
constexpr int kBNDec = 32;
constexpr int kDecStages = 3;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64, 2) void fwd_decode_kernel(const FwdArgs a) {
  constexpr int BN = kBNDec;
  constexpr int CPR = D / 8;
  constexpr int ROW = CPR * 16;
  constexpr int TILE = BN * ROW;
  constexpr int NQC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int DMA = TILE / (16 * 64);
  constexpr int NST = kDecStages;             // tile j read, j + 1 and j + 2 in flight
  constexpr int OFF_V = NST * TILE;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];

  const int lane = threadIdx.x;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int Nq = a.Nq, Nk = a.Nk, koff = a.koff;
  const float c = a.c;
  const int R = a.group * Nq;                 // packed rows of this head's group
  const int kvh = blockIdx.x / a.nsplit;      // b * Hkv + key/value head
  const int sp = blockIdx.x - kvh * a.nsplit;
  const bool live = n < R;
  const int g = live ? n / Nq : 0;            // query head within the group
  const int pos = live ? n - g * Nq : 0;      // query position
  const int bh = kvh * a.group + g;           // b * H + query head
  const size_t qoff = ((size_t)bh * Nq + pos) * D;
  const size_t kvbase = (size_t)kvh * (size_t)Nk * D;
  const char* Kb = reinterpret_cast<const char*>(a.K + kvbase);
  const char* Vb = reinterpret_cast<const char*>(a.V + kvbase);

  const int kb = sp * a.klen;
  const int ke = min(Nk, kb + a.klen);
  const int nkt = ke > kb ? (ke - kb + BN - 1) / BN : 0;

  const unsigned ldsb = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw));
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int k0 = kb + t * BN;
    const char* gk = Kb + (size_t)k0 * ROW;
    const char* gv = Vb + (size_t)k0 * ROW;
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const int slot = i * 64 + lane;
      const int row = slot / CPR;
      const int src_row = min(k0 + row, Nk - 1) - k0;
      const int ck = (slot % CPR) ^ swz<CPR, SWZ_ROWS>(row);
      const int cv = (slot % CPR) ^ swz<CPR, SWZ_TR>(row);
      dma16(gk, (unsigned)(src_row * ROW + ck * 16), ldsb + (t % NST) * TILE + i * 1024);
      dma16(gv, (unsigned)(src_row * ROW + cv * 16), ldsb + OFF_V + (t % NST) * TILE + i * 1024);
    }
  };
  if (nkt > 0) issue(0);
  if (nkt > 1) issue(1);

  bf16x8 qf[NQC];
  {
    const uint32_t flip = a.negq ? 0x80008000u : 0u;
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (live) raw = *reinterpret_cast<const u32x4*>(a.Q + qoff + 16 * cc + 8 * h);
      raw ^= flip;
      qf[cc] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const int ka = tile_off<CPR, SWZ_ROWS>(n, 8 * h);
  const int vrow0 = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int vcol0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int va = tile_off<CPR, SWZ_TR>(vrow0, vcol0);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kMInit;
  float lsum = 0.f;
  // last key this lane's row sees (rows past R see nothing)
  const int last = live ? (CAUSAL ? min(ke - 1, pos + koff) : ke - 1) : -1;

  for (int j = 0; j < nkt; ++j) {
    // tile j landed (the DMAs complete in order; tile j + 1's may still fly),
    // and tile j - 1, whose stage tile j + 2 takes, was read last round
    if (j + 1 < nkt)
      wait_vmem_but<2 * DMA>();
    else
      wait_vmem();
    if (j + 2 < nkt) issue(j + 2);
    const char* ks = smem_raw + (j % NST) * TILE;
    const char* vs = smem_raw + OFF_V + (j % NST) * TILE;
    const int k0 = kb + j * BN;

    f32x16 s = {};
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (ka ^ (32 * cc)));
      s = mfma_32x32x16_bf16(kf, qf[cc], s);
    }
    {
      const int lim = last - k0 - 4 * h;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        s[r] = off > lim ? kNegInf : s[r];
      }
    }
    uint32_t pk[8];
    auto probs = [&]() __attribute__((always_inline)) {
      float part[2] = {0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], c, -m));
        pk[r >> 1] = pack_bf16x2(p0, p1);
        part[(r >> 1) & 1] += p0 + p1;
      }
      return part[0] + part[1];
    };
    float ps = probs();
    if (__any(ps > kSumBound)) {
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      lsum *= alpha;
      m = m_new;
      ps = probs();
    }
    lsum += ps;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]});
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* vp = vs + (va ^ (64 * db)) + 16 * half * ROW;
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 8 * ROW);
        acc[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}),
                                     b, acc[db]);
      }
    }
  }

  const float lt = lsum + wave_xor32(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  if (live) {
    if (a.nsplit == 1) {
      uint16_t* orow = a.O + qoff;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int d0 = 32 * db + 8 * gg + 4 * h;
          u32x2 out = {pack_bf16x2(acc[db][4 * gg + 0] * inv, acc[db][4 * gg + 1] * inv),
                       pack_bf16x2(acc[db][4 * gg + 2] * inv, acc[db][4 * gg + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = out;
        }
      if (h == 0) a.LSE[(size_t)bh * Nq + pos] = lse;
    } else {
      const size_t prow = ((size_t)sp * a.BH + bh) * Nq + pos;
      float* orow = a.Opart + prow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int d0 = 32 * db + 8 * gg + 4 * h;
          f32x4 out = {acc[db][4 * gg + 0] * inv, acc[db][4 * gg + 1] * inv,
                       acc[db][4 * gg + 2] * inv, acc[db][4 * gg + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + d0) = out;
        }
      if (h == 0) a.Lpart[prow] = lse;
    }
  }
}

// Merge of the key ranges ("Flash Attention, From First Principles", "The
// scaffold": blocks over disjoint keys combine through their log-sum-exps):
// lse = log sum_s e^{lse_s}, O = sum_s e^{lse_s - lse} O_s.  Ranges with
// lse_s = -inf weigh 0; a row with no visible key at all keeps O = 0 and
// lse = -inf.  A row's D / 8 feature threads are repeated over 2^sg_log2
// split groups (split s to group s mod 2^sg_log2) whose maxima, weights and
// weighted sums are combined through LDS: with many splits (the decode's
// ranges) one thread per row would walk them all, one latency after another.
template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const float* __restrict__ Opart,
                                                        const float* __restrict__ Lpart,
                                                        uint16_t* __restrict__ O,
                                                        float* __restrict__ LSE, int rows,
                                                        int nsplit, int sg_log2) {
  constexpr int TPR = D / 8;
  __shared__ float red[256 * 9];
  const int SG = 1 << sg_log2;
  const int per_row = TPR << sg_log2;   // threads per row (<= 256)
  const int t = threadIdx.x;
  const int lr = t / per_row;
  const int sg = (t - lr * per_row) / TPR;
  const int part = t % TPR;
  const size_t row = (size_t)blockIdx.x * (256 / per_row) + lr;
  const bool live = row < (size_t)rows;
  float mx = kNegInf;
  if (live)
    for (int s = sg; s < nsplit; s += SG) mx = fmaxf(mx, Lpart[(size_t)s * rows + row]);
  red[t] = mx;
  __syncthreads();
  float gmx = kNegInf;
  for (int g = 0; g < SG; ++g) gmx = fmaxf(gmx, red[lr * per_row + g * TPR]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (live && gmx != kNegInf) {
    for (int s = sg; s < nsplit; s += SG) {
      const float wgt = __expf(Lpart[(size_t)s * rows + row] - gmx);
      den += wgt;
      const f32x4* src = reinterpret_cast<const f32x4*>(Opart + ((size_t)s * rows + row) * D +
                                                        part * 8);
      const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += wgt * x0[i];
        acc[4 + i] += wgt * x1[i];
      }
    }
  }
  __syncthreads();   // every thread has read the maxima
  red[9 * t] = den;
#pragma unroll
  for (int i = 0; i < 8; ++i) red[9 * t + 1 + i] = acc[i];
  __syncthreads();
  if (!live || sg != 0) return;
  for (int g = 1; g < SG; ++g) {
    const float* o = red + 9 * (lr * per_row + g * TPR + part);
    den += o[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += o[1 + i];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  u32x4 out = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
               pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4*>(O + row * D + part * 8) = out;
  if (part == 0) LSE[row] = den > 0.f ? gmx + __logf(den) : kNegInf;
}

// ---------------------------------------------------------------------------
// fp32 end to end: same schedule on the fp32 matrix cores (32x32x2), 32-key
// tiles, V kept row-major (each fp32 MFMA step needs one key per lane half).
// ---------------------------------------------------------------------------
template <int D>
struct FwdF32Cfg {
  static constexpr int BN = 32;
  static constexpr int RS = D + 4;            // row stride (floats), +16 B pad
  static constexpr int TILE = BN * RS;        // one K or V tile
  static constexpr int STAGE = 2 * TILE;      // K then V
  static constexpr int SMEM_BYTES = 2 * STAGE * 4;
  static constexpr int NDB = D / 32;
  static constexpr int LOADS = BN * D / 4 / 256;  // 16-byte chunks per thread per tensor
  static_assert(LOADS * 256 * 4 == BN * D, "f32 tile split");
};

template <int D>
struct TileRegsF32 {
  f32x4 k[FwdF32Cfg<D>::LOADS];
  f32x4 v[FwdF32Cfg<D>::LOADS];
};

template <int D>
__device__ __forceinline__ void load_tile_f32(TileRegsF32<D>& r, const float* __restrict__ Kh,
                                              const float* __restrict__ Vh, int k0, int N, int tid) {
  using C = FwdF32Cfg<D>;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int ci = i * 256 + tid;
    const int row = ci / (D / 4);
    const int col = (ci % (D / 4)) * 4;
    const int key = k0 + row;
    if (key < N) {
      r.k[i] = *reinterpret_cast<const f32x4*>(Kh + (size_t)key * D + col);
      r.v[i] = *reinterpret_cast<const f32x4*>(Vh + (size_t)key * D + col);
    } else {
      r.k[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      r.v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile_f32(const TileRegsF32<D>& r, float* stage, int tid) {
  using C = FwdF32Cfg<D>;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int ci = i * 256 + tid;
    const int row = ci / (D / 4);
    const int col = (ci % (D / 4)) * 4;
    *reinterpret_cast<f32x4*>(stage + row * C::RS + col) = r.k[i];
    *reinterpret_cast<f32x4*>(stage + C::TILE + row * C::RS + col) = r.v[i];
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqt, float c, int negq) {
  using C = FwdF32Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) float smemf[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;

  int bh, qt;
  map_tile(blockIdx.x, BH, nqt, CAUSAL, &bh, &qt);
  const size_t base = (size_t)bh * (size_t)N * D;
  const float* Qh = Q + base;
  const float* Kh = K + base;
  const float* Vh = V + base;
  const int q0 = qt * kBMF32;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + n;

  // B operand of S^T = K Q^T: lane holds Q[qrow][2i + h]
  float qf[D / 2];
#pragma unroll
  for (int i = 0; i < D / 2; ++i) {
    float x = (qrow < N) ? Qh[(size_t)qrow * D + 2 * i + h] : 0.f;
    qf[i] = negq ? -x : x;
  }

  const int kend = CAUSAL ? min(N, q0 + kBMF32) : N;
  const int nkt = (kend + C::BN - 1) / C::BN;

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kNegInf;
  float lsum = 0.f;

  TileRegsF32<D> regs;
  if (nkt > 0) {
    load_tile_f32<D>(regs, Kh, Vh, 0, N, tid);
    store_tile_f32<D>(regs, smemf, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * C::BN;
    const bool more = kt + 1 < nkt;
    if (more) load_tile_f32<D>(regs, Kh, Vh, k0 + C::BN, N, tid);
    const float* ks = smemf + (kt & 1) * C::STAGE;
    const float* vs = ks + C::TILE;

    const bool active = !CAUSAL || k0 <= wq0 + 31;
    if (active) {
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
      const float* krow = ks + n * C::RS + h;
#pragma unroll
      for (int i = 0; i < D / 2; ++i) s = mfma_32x32x2_f32(krow[2 * i], qf[i], s);

      if ((k0 + C::BN > N) || (CAUSAL && k0 + C::BN - 1 > wq0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
          bool dead = key >= N;
          if (CAUSAL) dead = dead || key > qrow;
          if (dead) s[r] = kNegInf;
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m, mx * c);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      float p[16];
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m_use));
        ps += p[r];
      }
      lsum = lsum * alpha + ps;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m = m_new;
      // O^T += V^T P^T: step r pairs key 8(r/4)+r%4 (lanes h=0) with key +4 (h=1)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          acc[db] = mfma_32x32x2_f32(vs[key * C::RS + 32 * db + n], p[r], acc[db]);
      }
    }
    if (more) store_tile_f32<D>(regs, smemf + ((kt + 1) & 1) * C::STAGE, tid);
    __syncthreads();
  }

  const float lt = lsum + wave_xor32(lsum);
  const float inv = 1.f / lt;
  if (qrow < N) {
    float* orow = O + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        f32x4 out = {acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                     acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + d0) = out;
      }
    if (h == 0) LSE[(size_t)bh * N + qrow] = (m + __log2f(lt)) * kLn2;
  }
}

// fp32 with the keys split over the waves, for grids too small to fill the
// GPU (the single-head N = 256 workload is two 128-query tiles, eight SIMDs
// at work, bound by the fp32 matrix rate of each).  A workgroup owns 32
// queries; wave w of four takes key tiles w, w + 4, .. (each staged through
// its own LDS region, no barrier) with its own running max, sum and
// accumulator, the partial results of disjoint key sets; at the end the
// other waves hand theirs to wave 0 through LDS, which combines them by the
// merge law of composite blocks ("Flash Attention, From First Principles",
// "The scaffold"): the largest max, every part rescaled to it, one division.
// Single-head N = 256: 28 -> 14.5 us, 13.7 with the next tile read during
// the current one (eight waves per workgroup, two per SIMD, were slower:
// 16.8 us; four independent score chains per tile too: 15.0 us).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_f32_split_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqt, float c, int negq) {
  using C = FwdF32Cfg<D>;
  constexpr int WAVES = 4;
  constexpr int WTILE = 2 * C::TILE;              // a wave's K and V tile (floats)
  constexpr int PER = C::BN * D / 4 / 64;         // 16-byte chunks per lane per tensor
  extern __shared__ __attribute__((aligned(16))) float smemf[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;

  int bh, qt;
  map_tile(blockIdx.x, BH, nqt, CAUSAL, &bh, &qt);
  const size_t base = (size_t)bh * (size_t)N * D;
  const float* Qh = Q + base;
  const float* Kh = K + base;
  const float* Vh = V + base;
  const int q0 = qt * 32;
  const int qrow = q0 + n;

  float qf[D / 2];
#pragma unroll
  for (int i = 0; i < D / 2; ++i) {
    float x = (qrow < N) ? Qh[(size_t)qrow * D + 2 * i + h] : 0.f;
    qf[i] = negq ? -x : x;
  }
  const int kend = CAUSAL ? min(N, q0 + 32) : N;
  const int nkt = (kend + C::BN - 1) / C::BN;

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kNegInf;
  float lsum = 0.f;
  float* ks = smemf + w * WTILE;
  float* vs = ks + C::TILE;

  // the wave's next tile is read from global memory into registers while
  // the current one is computed (rows past N read as 0)
  f32x4 kreg[PER], vreg[PER];
  auto fetch = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * C::BN;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ci = i * 64 + lane;
      const int row = ci / (D / 4);
      const int col = (ci % (D / 4)) * 4;
      kreg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      vreg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k0 + row < N) {
        kreg[i] = *reinterpret_cast<const f32x4*>(Kh + (size_t)(k0 + row) * D + col);
        vreg[i] = *reinterpret_cast<const f32x4*>(Vh + (size_t)(k0 + row) * D + col);
      }
    }
  };
  if (w < nkt) fetch(w);
  for (int kt = w; kt < nkt; kt += WAVES) {
    const int k0 = kt * C::BN;
    // this wave's tile into its LDS region
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ci = i * 64 + lane;
      const int row = ci / (D / 4);
      const int col = (ci % (D / 4)) * 4;
      *reinterpret_cast<f32x4*>(ks + row * C::RS + col) = kreg[i];
      *reinterpret_cast<f32x4*>(vs + row * C::RS + col) = vreg[i];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the writes above are done
    __builtin_amdgcn_wave_barrier();
    if (kt + WAVES < nkt) fetch(kt + WAVES);

    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const float* krow = ks + n * C::RS + h;
#pragma unroll
    for (int i = 0; i < D / 2; ++i) s = mfma_32x32x2_f32(krow[2 * i], qf[i], s);
    if ((k0 + C::BN > N) || (CAUSAL && k0 + C::BN - 1 > q0)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
        bool dead = key >= N;
        if (CAUSAL) dead = dead || key > qrow;
        if (dead) s[r] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m, mx * c);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    float pr[16];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m_use));
      ps += pr[r];
    }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    m = m_new;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        acc[db] = mfma_32x32x2_f32(vs[key * C::RS + 32 * db + n], pr[r], acc[db]);
    }
    // the next tile overwrites this region: every lane's reads are done
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
  }

  // waves 1..3 publish (max, sum, accumulator) in the layout every wave
  // shares (lane = query, registers = features); wave 0 merges
  const float lt = lsum + wave_xor32(lsum);
  __syncthreads();   // every wave is past its last tile read
  float* part = smemf;                                    // [WAVES - 1][NDB * 16][64]
  float* stat = smemf + (WAVES - 1) * C::NDB * 16 * 64;   // [WAVES - 1][2][64]
  if (w > 0) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[((w - 1) * C::NDB * 16 + db * 16 + r) * 64 + lane] =
          acc[db][r];
    stat[((w - 1) * 2 + 0) * 64 + lane] = m;
    stat[((w - 1) * 2 + 1) * 64 + lane] = lt;
  }
  __syncthreads();
  if (w != 0) return;
  float mw[WAVES], lw[WAVES];
  mw[0] = m;
  lw[0] = lt;
#pragma unroll
  for (int v = 1; v < WAVES; ++v) {
    mw[v] = stat[((v - 1) * 2 + 0) * 64 + lane];
    lw[v] = stat[((v - 1) * 2 + 1) * 64 + lane];
  }
  float mm = mw[0];
#pragma unroll
  for (int v = 1; v < WAVES; ++v) mm = fmaxf(mm, mw[v]);
  float wt[WAVES];
  float den = 0.f;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) {
    wt[v] = mw[v] == kNegInf ? 0.f : exp2f(mw[v] - mm);   // a part that saw no key weighs 0
    den += wt[v] * lw[v];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  if (qrow < N) {
    float* orow = O + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        f32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float x = wt[0] * acc[db][r];
#pragma unroll
          for (int v = 1; v < WAVES; ++v)
            x += wt[v] * part[((v - 1) * C::NDB * 16 + db * 16 + r) * 64 + lane];
          out[e] = x * inv;
        }
        *reinterpret_cast<f32x4*>(orow + d0) = out;
      }
    if (h == 0) LSE[(size_t)bh * N + qrow] = den > 0.f ? (mm + __log2f(den)) * kLn2 : kNegInf;
  }
}

// Softmax scale in log2 units.  scale == 0 (uniform attention) uses a tiny
// positive factor instead so masked scores still map to -inf, never NaN:
// every finite score then rounds to the same exponent, 0.
inline void split_scale(float scale, float* c, int* negq) {
  *negq = scale < 0.f;
  float a = scale < 0.f ? -scale : scale;
  *c = a > 0.f ? a * kLog2e : 1e-30f;
}

hipError_t launch_merge(const FwdArgs& a, int d, hipStream_t stream);

template <int D, int BN, bool CAUSAL>
hipError_t launch_bf16(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, BN>;
  auto kern = fwd_bf16_kernel<D, BN, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.BH * a.nqt * a.nsplit), dim3(64 * kWaves), C::SMEM_BYTES, stream,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_merge(a, D, stream);
}

hipError_t launch_merge(const FwdArgs& a, int d, hipStream_t stream) {
  const size_t rows = (size_t)a.BH * a.Nq;
  // split groups: about four splits per thread, at most 256 threads per row
  const int tpr = d / 8;
  int sg_log2 = 0;
  while ((4 << sg_log2) < a.nsplit && (tpr << (sg_log2 + 1)) <= 256) ++sg_log2;
  const size_t rows_per_wg = 256 / ((size_t)tpr << sg_log2);
  const dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  if (d == 256)
    hipLaunchKernelGGL(fwd_merge_kernel<256>, grid, dim3(256), 0, stream, a.Opart, a.Lpart, a.O,
                       a.LSE, (int)rows, a.nsplit, sg_log2);
  else if (d == 128)
    hipLaunchKernelGGL(fwd_merge_kernel<128>, grid, dim3(256), 0, stream, a.Opart, a.Lpart, a.O,
                       a.LSE, (int)rows, a.nsplit, sg_log2);
  else
    hipLaunchKernelGGL(fwd_merge_kernel<64>, grid, dim3(256), 0, stream, a.Opart, a.Lpart, a.O,
                       a.LSE, (int)rows, a.nsplit, sg_log2);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_decode(const FwdArgs& a, hipStream_t stream) {
  constexpr int smem = 2 * kDecStages * kBNDec * D * 2;
  auto kern = fwd_decode_kernel<D, CAUSAL>;
  hipError_t e =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((a.BH / a.group) * a.nsplit), dim3(64), smem, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_merge(a, D, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_inorder(FwdArgs a, hipStream_t stream) {
  using C = IoCfg<D>;
  // issue-priority thresholds at a quarter, a half and three quarters of the
  // longest workgroup's rounds
  const int most = (min(a.Nk, a.klen) + kBNIO - 1) / kBNIO;
  a.prio1 = most / 4;
  a.prio2 = most / 2;
  a.prio3 = 3 * most / 4;
  a.pass = max(1, device_cus() / 8);
  auto kern = fwd_inorder_kernel<D, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.BH * a.nqt * a.nsplit), dim3(64 * kWavesIO), C::SMEM, stream,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_merge(a, D, stream);
}

template <bool CAUSAL>
hipError_t launch_d256(FwdArgs a, hipStream_t stream) {
  constexpr int smem = 4 * kBN256 * 256 * 2;
  a.pass = max(1, device_cus() / 8);
  if constexpr (CAUSAL) {
    // only where the plain grid is a single wave of workgroups (two per CU):
    // with more, the hardware's dispatch of the later ones balances the CUs
    // and the plain kernel is faster ([2, 16, 4096, 256]: 39.0 % against
    // 37.1 % of peak; [1, 16, 4096, 256]: 30.9 % against 36.7 %)
    if (a.nsplit == 1 && a.nqt >= 2 && a.nqt % 2 == 0 && a.Nk > 0 && a.koff >= 0 &&
        (long long)a.BH * a.nqt <= 2LL * device_cus()) {
      // balanced pairs of query tiles: two K / V stage sets, then the merge's
      // parked float32 output (4 x 32 rows x 256) and (max, sum) per lane
      constexpr int park = 4 * 32 * 256 * 4 + 4 * 64 * 8;
      constexpr int smem_pair = 2 * smem > park ? 2 * smem : park;
      static_assert(smem_pair <= 160 * 1024, "LDS budget");
      auto kp = fwd_d256_pair_kernel<true>;
      hipError_t e = hipFuncSetAttribute((const void*)kp,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, smem_pair);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kp, dim3(a.BH * (a.nqt / 2)), dim3(2 * 64 * kWaves256), smem_pair,
                         stream, a);
      return hipGetLastError();
    }
  }
  auto kern = fwd_d256_kernel<CAUSAL>;
  hipError_t e =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.BH * a.nqt * a.nsplit), dim3(64 * kWaves256), smem, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_merge(a, 256, stream);
}

template <bool CAUSAL>
hipError_t launch_fp8(FwdArgs a, float vscale, hipStream_t stream) {
  constexpr int smem = 4 * kBNF8 * 128;
  a.pass = max(1, device_cus() / 8);
  auto kern = fwd_fp8_kernel<CAUSAL>;
  hipError_t e =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.BH * a.nqt * a.nsplit), dim3(64 * kWavesF8), smem, stream, a,
                     vscale);
  e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_merge(a, 128, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                      int BH, int N, float scale, hipStream_t stream) {
  using C = FwdF32Cfg<D>;
  const int nqt = (N + kBMF32 - 1) / kBMF32;
  float c;
  int negq;
  split_scale(scale, &c, &negq);
  if ((long long)BH * nqt < device_cus()) {
    // too few 128-query tiles to fill the GPU: 32-query workgroups with the
    // keys split over their waves
    auto kern = fwd_f32_split_kernel<D, CAUSAL>;
    constexpr int W = 4;
    constexpr int smem = W * 2 * C::TILE * 4;
    static_assert(smem >= ((W - 1) * C::NDB * 16 * 64 + (W - 1) * 2 * 64) * 4, "merge staging");
    static_assert(smem <= 160 * 1024, "LDS budget");
    hipError_t e =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    const int nqt32 = (N + 31) / 32;
    hipLaunchKernelGGL(kern, dim3(BH * nqt32), dim3(64 * W), smem, stream, q, k, v, o, lse, BH,
                       N, nqt32, c, negq);
    return hipGetLastError();
  }
  auto kern = fwd_f32_kernel<D, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(BH * nqt), dim3(256), C::SMEM_BYTES, stream, q, k, v, o, lse, BH,
                     N, nqt, c, negq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                              void* ws, int BH, int Nq, int Nk, int d, int group, bool causal,
                              float scale, const FwdPlan& pl, hipStream_t stream) {
  FwdArgs a;
  a.Q = (const uint16_t*)q;
  a.K = (const uint16_t*)k;
  a.V = (const uint16_t*)v;
  a.O = (uint16_t*)o;
  a.LSE = lse;
  a.BH = BH;
  a.Nq = Nq;
  a.Nk = Nk;
  a.koff = Nk - Nq;
  const int bm = fwd_rows_per_tile(d);
  a.nqt = (Nq + bm - 1) / bm;
  a.group = group;
  split_scale(scale, &a.c, &a.negq);
  a.nsplit = pl.nsplit;
  a.klen = pl.nsplit > 1 ? pl.klen : (Nk > 0 ? Nk : 1);
  a.Opart = nullptr;
  a.Lpart = nullptr;
  if (a.nsplit > 1) {
    const size_t rows = (size_t)a.nsplit * BH * Nq;
    a.Opart = (float*)ws;
    a.Lpart = (float*)((char*)ws + (rows * d * 4 + 255) / 256 * 256);
  }
  if (pl.decode) {
    if (d == 128)
      return causal ? launch_decode<128, true>(a, stream) : launch_decode<128, false>(a, stream);
    return causal ? launch_decode<64, true>(a, stream) : launch_decode<64, false>(a, stream);
  }
  if (d == 256) return causal ? launch_d256<true>(a, stream) : launch_d256<false>(a, stream);
  if (d == 128)
    return causal ? launch_bf16<128, 64, true>(a, stream) : launch_bf16<128, 64, false>(a, stream);
  return causal ? launch_inorder<64, true>(a, stream) : launch_inorder<64, false>(a, stream);
}

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                          int BH, int N, int d, bool causal, float score_scale, float v_scale,
                          hipStream_t stream) {
  if (d != 128) return hipErrorInvalidValue;
  FwdArgs a;
  a.Q = (const uint16_t*)q;   // byte tensors; the kernel reads them as e4m3
  a.K = (const uint16_t*)k;
  a.V = (const uint16_t*)v;
  a.O = (uint16_t*)o;
  a.LSE = lse;
  a.Opart = nullptr;
  a.Lpart = nullptr;
  a.BH = BH;
  a.Nq = N;
  a.Nk = N;
  a.koff = 0;
  a.nqt = (N + kBMF8 - 1) / kBMF8;
  a.nsplit = 1;
  a.klen = N > 0 ? N : 1;
  a.group = 1;
  split_scale(score_scale, &a.c, &a.negq);
  return causal ? launch_fp8<true>(a, v_scale, stream) : launch_fp8<false>(a, v_scale, stream);
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int BH, int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_f32<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_f32<128, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch_f32<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_f32<64, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace fa
