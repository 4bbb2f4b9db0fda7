// Backward kernels: recompute the probability tiles from the saved
// log-sum-exp instead of storing them ("Flash Attention, From First
// Principles", "The backward pass -- resurrection"; "FlashAttention from
// scratch", Step 4 and Follow-up questions).
//
// Three launches on the caller's stream:
//   1. bwd_pre:   per row, L2 = lse * log2(e) and -D = -sum_c dO_c * O_c (fp32),
//                 into a workspace padded to 64 rows per head; zero the fp32 dQ
//                 accumulator.
//   2. bwd_main:  one workgroup per key tile of one (batch, head); each wave
//                 owns 32 keys and keeps K, V (as MFMA operands) and its dK, dV
//                 accumulators in registers for the whole kernel.  Blocks of 64
//                 queries stream past the resident key tile (Q, dO and the
//                 block's L2 / D arrive in LDS by DMA, two stages deep); per
//                 block a wave recomputes
//                   S  = Q K^T                 (MFMA, lane = key)
//                   P  = exp(scale*S - lse)    (masked -> 0)
//                   dV^T += dO^T P             (MFMA)
//                   dP = dO V^T                (MFMA)
//                   dS = P * (dP - D)
//                   dK^T += Q^T dS             (MFMA)
//                 and, at d = 64, writes dS (bf16) to LDS.  At the start of the next
//                 iteration each wave forms its share of dQ = dS K from the
//                 previous block's dS (double-buffered) and the key tile in LDS
//                 -- 32x32 blocks over all the tile's keys, one per wave on
//                 waves 0..3, so every dQ element has one writer per key
//                 tile -- and adds it, times
//                 scale, into the fp32 accumulator with hardware float
//                 atomics; one barrier per block suffices.  The atomics are
//                 the kernel's scarcest resource (measured: removing them
//                 takes a quarter off its time at d = 64, half at d = 128):
//                 their count, one per dQ element per key tile, is why the
//                 key tiles are as large as the registers allow.
//                 Query blocks wholly before the key tile are skipped under
//                 causal masking ("LLM Architecture Refresh [3]", section 7).
//                 With grouped-query heads a group's query heads may be dealt
//                 to several workgroups per key tile, which then write float32
//                 partial dK, dV that bwd_kv_reduce_kernel sums (after the
//                 key-tile kernel below).
//   3. bwd_dq:    dQ = bf16(accumulator) at d = 64; at d = 128 and 256 dQ has
//                 its own query-stationary pass (section 4) and bwd_main makes
//                 dK and dV only.
//
// The P and dS registers of the S / dP accumulators are already the B
// operands of dV^T and dK^T (keys across lanes, queries across registers).
// Every transposed A/B operand (dO^T, Q^T, K^T, dS with queries across lanes)
// is read from a row-major LDS tile with ds_read_b64_tr_b16; no tile is ever
// transposed in registers.
#include <algorithm>
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBQ = kBwdQueryBlock;  // queries per streamed block

inline size_t round256(size_t b) { return (b + 255) / 256 * 256; }
inline int pad_rows(int N) { return (N + kBQ - 1) / kBQ * kBQ; }

// ---------------------------------------------------------------------------
// 1. L2 = lse*log2(e), -D = -rowsum(dO * O); zero the dQ accumulator
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      float* __restrict__ L2,
                                                      float* __restrict__ Dv,
                                                      float* __restrict__ dQacc, int N, int Npad,
                                                      size_t prow) {
  constexpr int TPR = D / 8;  // threads per row, 8 features each
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t prow_id = gid / TPR;      // padded row index over all heads
  const int part = (int)(gid % TPR);
  float acc = 0.f;
  const size_t bh = prow_id / Npad;
  const int i = (int)(prow_id - bh * Npad);
  const bool live = prow_id < prow && i < N;
  if (live) {
    const size_t off = (bh * N + i) * D + part * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + off);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc += bf16_bits_to_float(a[k] & 0xffffu) * bf16_bits_to_float(b[k] & 0xffffu);
      acc += bf16_bits_to_float(a[k] >> 16) * bf16_bits_to_float(b[k] >> 16);
    }
  }
  if (dQacc) {   // only the atomic (d = 64) path has an accumulator
    // the wave zeroes 512 consecutive elements as two contiguous 1 KiB runs
    // (a lane's own 8 elements as two 16-byte halves 16 bytes apart took
    // 0.6 us longer over the training-step shape)
    const size_t w0 = (gid - (gid & 63)) * 8;   // the wave's first element
    const size_t nel = (size_t)(prow / Npad) * N * D;
    const int ln = threadIdx.x & 63;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const size_t e = w0 + (size_t)u * 256 + 4 * ln;
      if (e < nel) *reinterpret_cast<f32x4*>(dQacc + e) = z;
    }
  }
#pragma unroll
  for (int s = TPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (prow_id < prow && part == 0) {
    Dv[prow_id] = live ? -acc : 0.f;   // -D: the dP accumulators start from it
    L2[prow_id] = live ? LSE[bh * N + i] * kLog2e : 0.f;
  }
}

// ---------------------------------------------------------------------------
// 3. dQ accumulator -> bf16
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ dQacc,
                                                     uint16_t* __restrict__ dQ, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(dQacc + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(dQacc + 8 * i + 4);
  u32x4 out = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
               pack_bf16x2(b[2], b[3])};
  *reinterpret_cast<u32x4*>(dQ + 8 * i) = out;
}

// ---------------------------------------------------------------------------
// 2. main kernel
// ---------------------------------------------------------------------------
template <int D>
struct BwdCfg {
  static constexpr int WAVES = D == 64 ? 8 : 4;   // d=64: 2 waves/SIMD; else 1
  // d = 64: dQ = dS K accumulated here with float atomics; d >= 128: dQ is
  // the query-stationary kernel's, this one makes dK and dV only (no K tile
  // or dS tile in LDS, no atomics)
  static constexpr bool DQA = (D == 64);
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int KEYS = 32 * WAVES;         // keys per workgroup
  static constexpr int CPRD = D / 8;              // 16-byte chunks per Q / dO / K row
  static constexpr int CPRQ = kBQ / 8;            // 16-byte chunks per dS row
  static constexpr int RBD = CPRD * 16;           // bytes per Q / dO / K row
  static constexpr int RBQ = CPRQ * 16;           // bytes per dS row
  static constexpr int NQS = kBQ / 32;            // 32-query sub-blocks
  static constexpr int NDC = D / 16;              // 16-feature chunks
  static constexpr int NDB = D / 32;              // 32-feature blocks
  static constexpr int QTILE = kBQ * D * 2;       // Q or dO tile (bytes)
  static constexpr int STAGE = 2 * QTILE + 2 * kBQ * 4;   // Q, dO, L2, D
  static constexpr int KTILE = KEYS * D * 2;
  static constexpr int DSTILE = KEYS * kBQ * 2;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_ST = DQA ? KTILE : 0;          // two stages
  static constexpr int OFF_DS = OFF_ST + 2 * STAGE;       // two dS buffers
  static constexpr int SMEM0 = OFF_DS + (DQA ? 2 * DSTILE : 0);
  // The K and V tiles go HBM -> LDS by DMA in whole rows and from there into
  // the operand registers, at OFF_KV (the dS buffers, idle until the first
  // dS write, or past them); head dimension 256 has no room and loads its
  // operands per lane.
  static constexpr int OFF_KV = OFF_DS;
  static constexpr bool KV_LDS = OFF_KV + 2 * KTILE <= 160 * 1024;
  static constexpr int SMEM = KV_LDS && OFF_KV + 2 * KTILE > SMEM0 ? OFF_KV + 2 * KTILE : SMEM0;
  static constexpr int QDMA = QTILE / 16 / THREADS;       // DMAs per thread per tile
  static constexpr int KDMA = KTILE / 16 / THREADS;
  // dQ = dS K in 32x32 blocks of the [kBQ, D] tile, each over all the tile's
  // keys, so every dQ element has one owner (two waves adding into the same
  // lines at once cost more than the rest of the kernel).  d = 64: the four
  // blocks go to waves 0..3, one per SIMD (16x16 blocks on all eight waves
  // read twice the LDS bytes per product); d = 128: two blocks per wave.
  static constexpr int NBLK = NQS * NDB;
  static constexpr int DQW = WAVES >= NBLK ? NBLK : WAVES;   // waves owning dQ blocks
  static constexpr int BPW = NBLK / DQW;                     // blocks per owner
  static_assert(QDMA * THREADS * 16 == QTILE && KDMA * THREADS * 16 == KTILE, "DMA split");
  static_assert(BPW * DQW == NBLK, "dQ block split");
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert(KEYS == bwd_keys_per_tile(D), "plan geometry");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(BwdCfg<D>::THREADS, 1) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ L2, const float* __restrict__ Dv, float* __restrict__ dQacc,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, float* __restrict__ part, int BHkv,
    int Nq, int Nk, int koff, int Npad, int nkt, int group, int hsplit, float scale, float c2) {
  using C = BwdCfg<D>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;

  // The workgroup owns a key tile of one key / value head; with grouped-query
  // attention the query heads sharing it are processed one after the other,
  // so dK and dV sum over them in registers (group = 1: plain multi-head
  // attention).  With hsplit > 1 the group's heads are dealt to hsplit
  // workgroups (group / hsplit each), which write float32 partial sums for a
  // reduction kernel instead of dK and dV.
  int unit, kt;
  map_tile(blockIdx.x, BHkv * hsplit, nkt, false, &unit, &kt);
  const int kvh = unit / hsplit;
  const int hpart = unit - kvh * hsplit;
  const int gsize = group / hsplit;
  const size_t kvbase = (size_t)kvh * (size_t)Nk * D;
  const char* Kb = reinterpret_cast<const char*>(K + kvbase);
  const char* Vb = reinterpret_cast<const char*>(V + kvbase);
  // per query head g of this workgroup's share: its Q, dO, L2, D and dQ
  // accumulator slice
  auto qhead = [&](int g) { return (size_t)kvh * group + hpart * gsize + g; };
  auto Qb_of = [&](int g) {
    return reinterpret_cast<const char*>(Q + qhead(g) * (size_t)Nq * D);
  };
  auto dOb_of = [&](int g) {
    return reinterpret_cast<const char*>(dO + qhead(g) * (size_t)Nq * D);
  };
  auto dq_rsrc_of = [&](int g) {
    return __builtin_amdgcn_make_buffer_rsrc(dQacc + qhead(g) * (size_t)Nq * D, (short)0,
                                             (int)((unsigned)Nq * (unsigned)D * 4u), 0x00020000);
  };

  const int k0 = kt * C::KEYS;
  const int wk0 = k0 + 32 * w;   // this wave's first key
  const int key = wk0 + n;       // this lane's key
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

  // key tile (row-major) for the K^T operand of dQ, read transposing by 16-
  // and 32-lane groups whose rows lie 8 apart: SWZ_BOTH keeps them apart
#pragma unroll
  for (int j = 0; j < (C::DQA ? C::KDMA : 0); ++j) {
    const int slot = (j * C::WAVES + w) * 64 + lane;
    const int row = slot / C::CPRD;
    const int chunk = (slot % C::CPRD) ^ swz<C::CPRD, SWZ_BOTH>(row);
    const int src = min(k0 + row, Nk - 1);
    dma16(Kb, (unsigned)((src * D + chunk * 8) * 2), lds0 + C::OFF_K + (j * C::WAVES + w) * 1024);
  }

  // Query i sees key j iff j <= i + koff (koff = Nk - Nq: the queries are the
  // last Nq positions).  Under causal masking the first query block that
  // sees any key of the tile is the one holding query k0 - koff.
  const int nqb = (Nq + kBQ - 1) / kBQ;
  const int qb0 = CAUSAL ? max(0, k0 - koff) / kBQ : 0;
  const int nit = max(0, nqb - qb0);   // query blocks per query head
  const int ntot = gsize * nit;    // iterations: (query head, query block)

  // DMA of iteration t: query block qb0 + t % nit of query head t / nit (Q, dO
  // rows clamped to N-1; L2 and D padded)
  auto issue = [&](int t) {
    const int g = t / nit;
    const int q0 = (qb0 + (t - g * nit)) * kBQ;
    const char* Qb = Qb_of(g);
    const char* dOb = dOb_of(g);
    const float* L2h = L2 + qhead(g) * Npad;
    const float* Dh = Dv + qhead(g) * Npad;
    const unsigned st = lds0 + C::OFF_ST + (t & 1) * C::STAGE;
    const int ln = D == 256 ? opaque(lane) : lane;
#pragma unroll
    for (int j = 0; j < C::QDMA; ++j) {
      const int slot = (j * C::WAVES + w) * 64 + ln;
      const int row = slot / C::CPRD;
      const int chunk = (slot % C::CPRD) ^ swz<C::CPRD, SWZ_BOTH>(row);
      const int src = min(q0 + row, Nq - 1);
      const unsigned off = (unsigned)((src * D + chunk * 8) * 2);
      dma16(Qb, off, st + (j * C::WAVES + w) * 1024);
      dma16(dOb, off, st + C::QTILE + (j * C::WAVES + w) * 1024);
    }
    if (w == 0) {
      if (lane < 16)
        dma16(L2h + q0, lane * 16, st + 2 * C::QTILE);
      else if (lane < 32)
        dma16(Dh + q0, (lane - 16) * 16, st + 2 * C::QTILE);
    }
  };
  if (ntot > 0) issue(0);

  // K and V as B operands (lane = key, 8 consecutive features per chunk)
  bf16x8 kf[C::NDC], vf[C::NDC];
  if constexpr (C::KV_LDS) {
    // whole-row DMA (row swizzle; rows past Nk fall outside the buffer
    // resource and read 0), then 16-byte LDS reads: per-lane loads straight
    // from HBM would touch 32 rows per instruction.  Wave w fills slots
    // w, w + WAVES, ..; DMA j + 1 is DMA j shifted by WAVES KiB on both sides,
    // a multiple of the swizzle's 16-row period.
    static_assert((C::WAVES * 1024 / C::RBD) % 16 == 0, "swizzle period");
    const int slot = w * 64 + lane;
    const int row = slot / C::CPRD;
    const unsigned off =
        (unsigned)((row * D + ((slot % C::CPRD) ^ swz<C::CPRD, SWZ_ROWS>(row)) * 8) * 2);
    const long long kbytes = (long long)max(0, Nk - k0) * (D * 2);
#pragma unroll
    for (int j = 0; j < C::KDMA; ++j) {
      const long long b0 = (long long)j * C::WAVES * 1024;
      const long long nrec = kbytes - b0 > 0 ? kbytes - b0 : 0;
      const unsigned dst = lds0 + C::OFF_KV + (unsigned)b0 + w * 1024;
      dma16_buf(__builtin_amdgcn_make_buffer_rsrc((void*)(Kb + (size_t)k0 * D * 2 + b0), (short)0,
                                                  (int)nrec, 0x00020000),
                off, dst);
      dma16_buf(__builtin_amdgcn_make_buffer_rsrc((void*)(Vb + (size_t)k0 * D * 2 + b0), (short)0,
                                                  (int)nrec, 0x00020000),
                off, dst + C::KTILE);
    }
    wait_vmem();
    __syncthreads();
    const char* kvs = smem + C::OFF_KV + 32 * w * C::RBD;
#pragma unroll
    for (int cc = 0; cc < C::NDC; ++cc) {
      const int o = tile_off<C::CPRD, SWZ_ROWS>(n, 16 * cc + 8 * h);
      kf[cc] = *reinterpret_cast<const bf16x8*>(kvs + o);
      vf[cc] = *reinterpret_cast<const bf16x8*>(kvs + C::KTILE + o);
    }
  } else {
#pragma unroll
    for (int cc = 0; cc < C::NDC; ++cc) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key < Nk) {
        a = *reinterpret_cast<const u32x4*>(Kb + ((size_t)key * D + 16 * cc + 8 * h) * 2);
        b = *reinterpret_cast<const u32x4*>(Vb + ((size_t)key * D + 16 * cc + 8 * h) * 2);
      }
      kf[cc] = __builtin_bit_cast(bf16x8, a);
      vf[cc] = __builtin_bit_cast(bf16x8, b);
    }
  }

  // per-lane LDS offsets
  // row-operand reads of Q / dO (A of S and dP): row 32qs + n, features 16cc + 8h
  // (chunk index and swizzle occupy disjoint bits, so feature chunk cc / block
  // db is the cc = 0 / db = 0 offset XOR 32 cc / 64 db: two base registers
  // instead of an offset per chunk; the per-chunk offsets are formed in the
  // query loop)
  const int qro0 = tile_off<C::CPRD, SWZ_BOTH>(n, 8 * h);
  // transposing reads: 16-lane group g reads rows 4*(g/2) + j (+8 for the
  // second read) and columns 16*(g%2) + 4*(lane%4) of a 32-column block
  const int trow = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // dO^T / Q^T A operands (rows = queries): rows trow and trow + 8
  const int qtr0 = tile_off<C::CPRD, SWZ_BOTH>(trow, tcol);
  const int qtr1 = tile_off<C::CPRD, SWZ_BOTH>(trow + 8, tcol);
  // dS writes: row 32w + n (this lane's key), queries 32qs + 8g + 4h .. +3.
  // The dS tile is row-written and transposing-read, so it uses SWZ_BOTH; its
  // chunk positions are not affine in g, hence one offset per (qs, g).
  int dsw[C::NQS][4];
#pragma unroll
  for (int qs = 0; qs < C::NQS; ++qs)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      dsw[qs][g] = tile_off<C::CPRQ, SWZ_BOTH>(32 * w + n, 32 * qs + 8 * g + 4 * h);

  f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  // dQ = dS K for query block it, from dS buffer it & 1, added (times scale)
  // into the fp32 accumulator with buffer atomics: one per-lane offset, the
  // register's row as a uniform offset; all rows valid is the common,
  // branch-free case.  Key chunks past the causal limit hold dS = 0 (masked
  // P, or zeros written by waves with no visible key), so the k loop is
  // straight-line and only a block with no visible key at all is skipped.
  auto dq_step = [&](int t) {
    if (!C::DQA || w >= C::DQW) return;
    const int gq = t / nit;
    const int q0 = (qb0 + (t - gq * nit)) * kBQ;
    const __amdgpu_buffer_rsrc_t dq_rsrc = dq_rsrc_of(gq);
    const char* dsb = smem + C::OFF_DS + (t & 1) * C::DSTILE;
    const char* kt_lds = smem + C::OFF_K;
#pragma unroll
    for (int bi = 0; bi < C::BPW; ++bi) {
      const int blk = w * C::BPW + bi;
      const int qsq = blk / C::NDB;
      const int dbq = blk % C::NDB;
      const int qs0 = q0 + 32 * qsq;
      if (CAUSAL && k0 > qs0 + 31 + koff) continue;
      // SWZ_BOTH depends on row bits 1..3: the two 8-row halves differ
      const int aoff0 = tile_off<C::CPRQ, SWZ_BOTH>(trow, 32 * qsq + tcol);
      const int aoff1 = tile_off<C::CPRQ, SWZ_BOTH>(trow + 8, 32 * qsq + tcol);
      const int boff0 = tile_off<C::CPRD, SWZ_BOTH>(trow, 32 * dbq + tcol);
      const int boff1 = tile_off<C::CPRD, SWZ_BOTH>(trow + 8, 32 * dbq + tcol);
      f32x16 acc = {};
#pragma unroll
      for (int kc = 0; kc < C::KEYS / 16; ++kc) {
        const u32x2 a0 = lds_read_tr16(dsb + aoff0 + (16 * kc) * C::RBQ);
        const u32x2 a1 = lds_read_tr16(dsb + aoff1 + (16 * kc) * C::RBQ);
        const u32x2 b0 = lds_read_tr16(kt_lds + boff0 + (16 * kc) * C::RBD);
        const u32x2 b1 = lds_read_tr16(kt_lds + boff1 + (16 * kc) * C::RBD);
        acc = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y}),
                                 __builtin_bit_cast(bf16x8, u32x4{b0.x, b0.y, b1.x, b1.y}),
                                 acc);
      }
      // acc: lane = feature 32*dbq + n, registers = queries qs0 + 4h + 8(r/4) + r%4
      const int voff = ((qs0 + 4 * h) * D + 32 * dbq + n) * 4;
      if (qs0 + 31 < Nq) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
              scale * acc[r], dq_rsrc, voff, (8 * (r >> 2) + (r & 3)) * D * 4, 0);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = qs0 + 4 * h + 8 * (r >> 2) + (r & 3);
          if (qrow < Nq)
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                scale * acc[r], dq_rsrc, voff, (8 * (r >> 2) + (r & 3)) * D * 4, 0);
        }
      }
    }
  };

  for (int t = 0; t < ntot; ++t) {
    const int q0 = (qb0 + (t % nit)) * kBQ;
    // stage t landed for every lane; every wave is done with iteration t-1
    wait_vmem();
    __syncthreads();
    if (t + 1 < ntot) issue(t + 1);
    if (C::DQA && t > 0) dq_step(t - 1);

    const char* st = smem + C::OFF_ST + (t & 1) * C::STAGE;
    const char* sQ = st;
    const char* sdO = st + C::QTILE;
    const float* sL2 = reinterpret_cast<const float*>(st + 2 * C::QTILE);
    const float* sD = sL2 + kBQ;
    char* dsb = smem + C::OFF_DS + (t & 1) * C::DSTILE;

    // (d = 256 without causal masking: one sub-block body, not two copies --
    // the copies left the register allocator a few registers short)
    constexpr int kQsUnroll = D == 256 && !CAUSAL ? 1 : C::NQS;
#pragma unroll kQsUnroll
    for (int qs = 0; qs < C::NQS; ++qs) {
      const int qs0 = q0 + 32 * qs;
      // d = 256: the operand offsets are recomputed from their bases here
      const int qro0_ = D == 256 ? opaque(qro0) : qro0;
      const int qtr0_ = D == 256 ? opaque(qtr0) : qtr0;
      const int qtr1_ = D == 256 ? opaque(qtr1) : qtr1;
      auto qro = [&](int cc) __attribute__((always_inline)) { return qro0_ ^ (32 * cc); };
      auto qtr = [&](int db, int rd) __attribute__((always_inline)) {
        return (rd ? qtr1_ : qtr0_) ^ (64 * db);
      };
      uint32_t sk[8];
      // the wave's keys all come after every query of the sub-block: dS = 0
      const bool dead = CAUSAL && (wk0 > qs0 + 31 + koff);
      if (!dead) {
        // registers r: query qs0 + 4h + off, off = 8(r/4) + r%4; lane = key.
        // L2 of register group g (four queries) is read where used; the dP
        // accumulator starts from -D of each register's query, so the
        // products leave dP - D in it and dS = P (dP - D) is one multiply
        auto l2_of = [&](int g) __attribute__((always_inline)) {
          return *reinterpret_cast<const f32x4*>(sL2 + 32 * qs + 8 * g + 4 * h);
        };
        auto nd_of = [&](int g) __attribute__((always_inline)) {
          return *reinterpret_cast<const f32x4*>(sD + 32 * qs + 8 * g + 4 * h);
        };
        f32x16 s = {};
        f32x16 dp;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 nd = nd_of(g);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * g + e] = nd[e];
        }
#pragma unroll
        for (int cc = 0; cc < C::NDC; ++cc) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQ + qro(cc) + 32 * qs * C::RBD);
          const bf16x8 ag = *reinterpret_cast<const bf16x8*>(sdO + qro(cc) + 32 * qs * C::RBD);
          s = mfma_32x32x16_bf16(aq, kf[cc], s);
          dp = mfma_32x32x16_bf16(ag, vf[cc], dp);
        }
        const bool need_mask =
            (qs0 + 31 >= Nq) || (wk0 + 31 >= Nk) || (CAUSAL && wk0 + 31 > qs0 + koff);
        int lo = -1, hi = 1 << 30;   // live offsets: lo < off+1 ... i.e. off >= lo, off < hi
        if (need_mask) {
          if (CAUSAL) lo = key - koff - qs0 - 4 * h;
          hi = key < Nk ? Nq - qs0 - 4 * h : -(1 << 30);
        }
        uint32_t pk[8];
        // P and dS; the mask compares exist only in the masked instance (a
        // branch-free select in every sub-block cost 4 VALU ops per score)
        auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 l2v = l2_of(g);
#pragma unroll
            for (int r = 4 * g; r < 4 * g + 4; r += 2) {
              float p2[2], ds2[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int rr = r + u;
                const int off = 8 * (rr >> 2) + (rr & 3);
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], c2, -l2v[rr & 3]));
                if constexpr (decltype(masked)::value) p = (off < lo || off >= hi) ? 0.f : p;
                p2[u] = p;
                ds2[u] = p * dp[rr];
              }
              pk[r >> 1] = pack_bf16x2(p2[0], p2[1]);
              sk[r >> 1] = pack_bf16x2(ds2[0], ds2[1]);
            }
          }
        };
        if (need_mask)
          probs(std::true_type{});
        else
          probs(std::false_type{});
        // dV^T += dO^T P ; dK^T += Q^T dS  (k = the 16 queries of one half)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8 bp = __builtin_bit_cast(
              bf16x8, u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]});
          const bf16x8 bs = __builtin_bit_cast(
              bf16x8, u32x4{sk[4 * half], sk[4 * half + 1], sk[4 * half + 2], sk[4 * half + 3]});
          const int rowoff = (32 * qs + 16 * half) * C::RBD;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const u32x2 g0 = lds_read_tr16(sdO + qtr(db, 0) + rowoff);
            const u32x2 g1 = lds_read_tr16(sdO + qtr(db, 1) + rowoff);
            const u32x2 q0v = lds_read_tr16(sQ + qtr(db, 0) + rowoff);
            const u32x2 q1v = lds_read_tr16(sQ + qtr(db, 1) + rowoff);
            dv[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{g0.x, g0.y, g1.x, g1.y}),
                                        bp, dv[db]);
            dk[db] = mfma_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, u32x4{q0v.x, q0v.y, q1v.x, q1v.y}), bs, dk[db]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) sk[i] = 0u;
      }
      // dS (bf16) into LDS as [key][query]: registers 4g..4g+3 are queries
      // 32qs + 8g + 4h .. +3
      if constexpr (C::DQA) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<u32x2*>(dsb + dsw[qs][g]) = u32x2{sk[2 * g], sk[2 * g + 1]};
      }
    }
  }
  if constexpr (C::DQA) {
    wait_vmem();
    __syncthreads();
    if (ntot > 0) dq_step(ntot - 1);
  }

  if (hsplit > 1) {
    // float32 partials [hsplit][BHkv][Nk][D] (dK, then dV): lane = key,
    // registers 4g..4g+3 = features 32 db + 8 g + 4 h .. + 3
    float* pk = part + ((size_t)hpart * BHkv + kvh) * (size_t)Nk * D;
    float* pv = pk + (size_t)hsplit * BHkv * (size_t)Nk * D;
    if (key < Nk) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const size_t o = (size_t)key * D + 32 * db + 8 * g + 4 * h;
          *reinterpret_cast<f32x4*>(pk + o) =
              f32x4{scale * dk[db][4 * g + 0], scale * dk[db][4 * g + 1],
                    scale * dk[db][4 * g + 2], scale * dk[db][4 * g + 3]};
          *reinterpret_cast<f32x4*>(pv + o) =
              f32x4{dv[db][4 * g + 0], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
        }
    }
    return;
  }

  // epilogue: dK = scale * dK^T acc, dV = dV^T acc (lane = key, registers =
  // features), through LDS so the stores are whole rows: every wave writes
  // its 32 x D blocks (row swizzle), then stores 16-byte chunks.
  // every wave is past its last LDS read (the dQ atomics may still fly)
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  {
    char* ks = smem + 32 * w * C::RBD;
    char* vs = ks + C::KTILE;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int o = tile_off<C::CPRD, SWZ_ROWS>(n, 32 * db + 8 * g + 4 * h);
        *reinterpret_cast<u32x2*>(ks + o) =
            u32x2{pack_bf16x2(scale * dk[db][4 * g + 0], scale * dk[db][4 * g + 1]),
                  pack_bf16x2(scale * dk[db][4 * g + 2], scale * dk[db][4 * g + 3])};
        *reinterpret_cast<u32x2*>(vs + o) =
            u32x2{pack_bf16x2(dv[db][4 * g + 0], dv[db][4 * g + 1]),
                  pack_bf16x2(dv[db][4 * g + 2], dv[db][4 * g + 3])};
      }
    constexpr int PER = 64 / C::CPRD;   // rows per store instruction
#pragma unroll
    for (int it = 0; it < 32 / PER; ++it) {
      const int r = it * PER + lane / C::CPRD, ch = lane % C::CPRD;
      const int o = tile_off<C::CPRD, SWZ_ROWS>(r, 8 * ch);
      const u32x4 kv16 = *reinterpret_cast<const u32x4*>(ks + o);
      const u32x4 vv16 = *reinterpret_cast<const u32x4*>(vs + o);
      if (wk0 + r < Nk) {
        *reinterpret_cast<u32x4*>(dK + kvbase + (size_t)(wk0 + r) * D + 8 * ch) = kv16;
        *reinterpret_cast<u32x4*>(dV + kvbase + (size_t)(wk0 + r) * D + 8 * ch) = vv16;
      }
    }
  }
}

// workspace layout: L2 [BH * Npad], -D [BH * Npad], dQ accumulator [BH * N * d]
struct WsLayout {
  float* l2;
  float* dv;
  float* dq;
};
inline WsLayout ws_layout(void* ws, int BH, int N) {
  char* p = reinterpret_cast<char*>(ws);
  const size_t rows = round256((size_t)BH * pad_rows(N) * 4);
  return WsLayout{reinterpret_cast<float*>(p), reinterpret_cast<float*>(p + rows),
                  reinterpret_cast<float*>(p + 2 * rows)};
}

template <int D, bool CAUSAL>
hipError_t launch_main(const void* q, const void* k, const void* v, const void* dout,
                       const WsLayout& w, void* dk, void* dv, float* part, int BH, int Nq, int Nk,
                       int group, int hsplit, float scale, hipStream_t stream) {
  using C = BwdCfg<D>;
  const int nkt = (Nk + C::KEYS - 1) / C::KEYS;
  const int BHkv = BH / group;
  auto kern = bwd_main_kernel<D, CAUSAL>;
  hipError_t e =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(BHkv * hsplit * nkt), dim3(C::THREADS), C::SMEM, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     (const uint16_t*)dout, w.l2, w.dv, w.dq, (uint16_t*)dk, (uint16_t*)dv, part,
                     BHkv, Nq, Nk, Nk - Nq, pad_rows(Nq), nkt, group, hsplit, scale,
                     scale * kLog2e);
  return hipGetLastError();
}

// dK, dV = bf16(sum of the hsplit float32 partials), summed in partial order
// (deterministic); one thread per 8 elements of each tensor.
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(const float* __restrict__ part,
                                                            uint16_t* __restrict__ dK,
                                                            uint16_t* __restrict__ dV, size_t n8,
                                                            int hsplit) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const size_t slice = n8 * 8;   // elements per partial
  const float* pk = part + 8 * i;
  const float* pv = pk + (size_t)hsplit * slice;
  f32x4 k0 = *reinterpret_cast<const f32x4*>(pk), k1 = *reinterpret_cast<const f32x4*>(pk + 4);
  f32x4 v0 = *reinterpret_cast<const f32x4*>(pv), v1 = *reinterpret_cast<const f32x4*>(pv + 4);
  for (int s = 1; s < hsplit; ++s) {
    k0 += *reinterpret_cast<const f32x4*>(pk + s * slice);
    k1 += *reinterpret_cast<const f32x4*>(pk + s * slice + 4);
    v0 += *reinterpret_cast<const f32x4*>(pv + s * slice);
    v1 += *reinterpret_cast<const f32x4*>(pv + s * slice + 4);
  }
  *reinterpret_cast<u32x4*>(dK + 8 * i) = u32x4{pack_bf16x2(k0[0], k0[1]), pack_bf16x2(k0[2], k0[3]),
                                                pack_bf16x2(k1[0], k1[1]), pack_bf16x2(k1[2], k1[3])};
  *reinterpret_cast<u32x4*>(dV + 8 * i) = u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                                                pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
}

// dK = dV = 0 when there are no queries (nothing to differentiate through).
__global__ __launch_bounds__(256) void zero_pair_kernel(uint32_t* __restrict__ a,
                                                        uint32_t* __restrict__ b, size_t n8) {
  // one thread per 8 bf16 (16 bytes) of each tensor
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4 z = {0u, 0u, 0u, 0u};
  reinterpret_cast<u32x4*>(a)[i] = z;
  reinterpret_cast<u32x4*>(b)[i] = z;
}

// ---------------------------------------------------------------------------
// 4. dQ without atomics (d = 128 and 256): query-stationary
// ---------------------------------------------------------------------------
// At d >= 128 the key-tile kernel's dQ float atomics cost more than all its
// matrix work (measured at d = 128: 860 us with them, 398 us without), so
// there dQ gets its own pass over the key tiles, the loop order of the
// forward: a workgroup owns 128 queries (4 waves x 32, one wave per SIMD) and
// streams the key / value tiles past them, recomputing per tile
//   S^T  = K Q^T,   dP^T = V dO^T       (MFMA; lane = query, as the forward)
//   P    = exp2(c2 S - L2),  dS = P (dP - D)
//   dQ^T += K^T dS^T                    (MFMA; dS^T already the B operand)
// and writes dQ = scale * dQ^T once, in bf16: 1.5x the matrix work of the
// key-tile kernel's dQ product ("FlashAttention from scratch", Follow-up
// questions: dQ accumulated separately from dK and dV).  The K tile is read
// both by rows (S) and transposed (dQ), so it uses the two-pattern swizzle;
// V is only read by rows.
template <int D>
struct DqCfg {
  static constexpr int WAVES = 4;
  static constexpr int QB = 32 * WAVES;
  static constexpr int BN = D == 256 ? 32 : 64;
  static constexpr int CPR = D / 8;
  static constexpr int ROW = CPR * 16;
  static constexpr int TILE = BN * ROW;
  static constexpr int NSB = BN / 32;
  static constexpr int NQC = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int DMA = TILE / (16 * 64 * WAVES);
  static constexpr int OFF_V = 2 * TILE;
  static constexpr int SMEM = 4 * TILE;
  static constexpr int QTILE = QB * ROW;        // the dQ tile, staged in the K/V stages
  static_assert(DMA * 16 * 64 * WAVES == TILE, "DMA split");
  static_assert(QTILE <= 4 * TILE, "the dQ tile fits the K/V stages");
};

// d = 128: two waves per SIMD (two workgroups per CU), so one workgroup's
// vector work overlaps the other's matrix work (297 -> 257 us at
// [1, 32, 4096, 128] causal); d = 256 needs more than 256 registers.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, D == 128 ? 2 : 1) void bwd_dq_direct_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ L2, const float* __restrict__ Dv, uint16_t* __restrict__ dQ,
    int BH, int Nq, int Nk, int koff, int Npad, int nqt, int group, float scale, float c2) {
  using C = DqCfg<D>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;

  int bh, qt;
  map_tile(blockIdx.x, BH, nqt, CAUSAL, &bh, &qt);
  const size_t qbase = (size_t)bh * (size_t)Nq * D;
  const size_t kvbase = (size_t)(bh / group) * (size_t)Nk * D;
  const char* Kb = reinterpret_cast<const char*>(K + kvbase);
  const char* Vb = reinterpret_cast<const char*>(V + kvbase);
  const int q0 = qt * C::QB;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + n;
  const int ke = CAUSAL ? min(Nk, q0 + C::QB + koff) : Nk;
  const int nkt = ke > 0 ? (ke + C::BN - 1) / C::BN : 0;

  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * C::BN;
    const char* gk = Kb + (size_t)k0 * C::ROW;
    const char* gv = Vb + (size_t)k0 * C::ROW;
#pragma unroll
    for (int i = 0; i < C::DMA; ++i) {
      const int slot = (i * C::WAVES + w) * 64 + lane;
      const int row = slot / C::CPR;
      const int src_row = min(k0 + row, Nk - 1) - k0;
      const int ck = (slot % C::CPR) ^ swz<C::CPR, SWZ_BOTH>(row);
      const int cv = (slot % C::CPR) ^ swz<C::CPR, SWZ_ROWS>(row);
      const unsigned dst = (unsigned)((i * C::WAVES + w) * 1024);
      dma16(gk, (unsigned)(src_row * C::ROW + ck * 16), lds0 + (t & 1) * C::TILE + dst);
      dma16(gv, (unsigned)(src_row * C::ROW + cv * 16), lds0 + C::OFF_V + (t & 1) * C::TILE + dst);
    }
  };
  if (nkt > 0) issue(0);

  // Q^T and dO^T as B operands: lane = query, features 16 cc + 8 h .. + 7
  bf16x8 qf[C::NQC], gf[C::NQC];
#pragma unroll
  for (int cc = 0; cc < C::NQC; ++cc) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (qrow < Nq) {
      a = *reinterpret_cast<const u32x4*>(Q + qbase + (size_t)qrow * D + 16 * cc + 8 * h);
      b = *reinterpret_cast<const u32x4*>(dO + qbase + (size_t)qrow * D + 16 * cc + 8 * h);
    }
    qf[cc] = __builtin_bit_cast(bf16x8, a);
    gf[cc] = __builtin_bit_cast(bf16x8, b);
  }
  const float l2 = qrow < Nq ? L2[(size_t)bh * Npad + qrow] : 0.f;
  const float nd = qrow < Nq ? Dv[(size_t)bh * Npad + qrow] : 0.f;   // -D of the query

  // row reads (A of S^T and dP^T): row 32 sb + n, chunk 2 cc + h
  const int ka0 = tile_off<C::CPR, SWZ_BOTH>(n, 8 * h);
  const int va0 = tile_off<C::CPR, SWZ_ROWS>(n, 8 * h);
  // transposing reads of the K tile (A of dQ^T = K^T dS^T), the forward's
  // V^T pattern: rows vrow0 (+ 8) of each 16-key chunk, columns 32 db + vcol0
  const int vrow0 = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int vcol0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int kt_lo0 = tile_off<C::CPR, SWZ_BOTH>(vrow0, vcol0);
  const int kt_hi0 = tile_off<C::CPR, SWZ_BOTH>(vrow0 + 8, vcol0);

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  for (int j = 0; j < nkt; ++j) {
    wait_vmem();
    __syncthreads();
    if (j + 1 < nkt) issue(j + 1);
    const char* ks = smem + (j & 1) * C::TILE;
    const char* vs = smem + C::OFF_V + (j & 1) * C::TILE;
    const int k0 = j * C::BN;
    // operand offsets recomputed from their bases each tile rather than held
    // (at two waves per SIMD the registers are short)
    const int ka = opaque(ka0), va = opaque(va0);
    const int kt_lo = opaque(kt_lo0), kt_hi = opaque(kt_hi0);

    f32x16 s[C::NSB], dp[C::NSB];
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
      s[sb] = f32x16{};
      dp[sb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < C::NQC; ++cc) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(ks + (ka ^ (32 * cc)) + 32 * sb * C::ROW);
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8*>(vs + (va ^ (32 * cc)) + 32 * sb * C::ROW);
        s[sb] = mfma_32x32x16_bf16(kf, qf[cc], s[sb]);
        dp[sb] = mfma_32x32x16_bf16(vf, gf[cc], dp[sb]);
      }
    }
    // register r of sub-block sb holds key k0 + 32 sb + 8 (r / 4) + 4 h + r % 4
    const bool masked = (k0 + C::BN > Nk) || (CAUSAL && k0 + C::BN - 1 > wq0 + koff);
    int lim = Nk - 1 - k0 - 4 * h;
    if (CAUSAL) lim = min(lim, qrow + koff - k0 - 4 * h);
    uint32_t dsk[C::NSB][8];
    auto form = [&](auto mk) __attribute__((always_inline)) {
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float d2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int rr = r + u;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][rr], c2, -l2));
            if constexpr (decltype(mk)::value) {
              const int off = 32 * sb + 8 * (rr >> 2) + (rr & 3);
              p = off > lim ? 0.f : p;   // select after the exp: l2 may be -inf
            }
            d2[u] = p * (dp[sb][rr] + nd);
          }
          dsk[sb][r >> 1] = pack_bf16x2(d2[0], d2[1]);
        }
    };
    if (masked)
      form(std::true_type{});
    else
      form(std::false_type{});

#pragma unroll
    for (int kc = 0; kc < C::BN / 16; ++kc) {
      const int sb = kc >> 1, half = kc & 1;
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, u32x4{dsk[sb][4 * half], dsk[sb][4 * half + 1], dsk[sb][4 * half + 2],
                        dsk[sb][4 * half + 3]});
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const u32x2 lo = lds_read_tr16(ks + (kt_lo ^ (64 * db)) + 16 * kc * C::ROW);
        const u32x2 hi = lds_read_tr16(ks + (kt_hi ^ (64 * db)) + 16 * kc * C::ROW);
        acc[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}),
                                     b, acc[db]);
      }
    }
  }

  // dQ through LDS (the K / V stages) so the stores are whole rows: every
  // wave writes its 32 x D block (row swizzle), then stores 16-byte chunks
  wait_vmem();
  __syncthreads();   // every wave is past its last LDS read
  char* os = smem + 32 * w * C::ROW;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * h;
      *reinterpret_cast<u32x2*>(os + tile_off<C::CPR, SWZ_ROWS>(n, d0)) =
          u32x2{pack_bf16x2(scale * acc[db][4 * g + 0], scale * acc[db][4 * g + 1]),
                pack_bf16x2(scale * acc[db][4 * g + 2], scale * acc[db][4 * g + 3])};
    }
  constexpr int PER = 64 / C::CPR;   // rows per store instruction
#pragma unroll
  for (int it = 0; it < 32 / PER; ++it) {
    const int r = it * PER + lane / C::CPR, ch = lane % C::CPR;
    const u32x4 v16 = *reinterpret_cast<const u32x4*>(os + tile_off<C::CPR, SWZ_ROWS>(r, 8 * ch));
    if (wq0 + r < Nq) *reinterpret_cast<u32x4*>(dQ + qbase + (size_t)(wq0 + r) * D + 8 * ch) = v16;
  }
}

}  // namespace

hipError_t launch_bwd_pre(const void* o, const void* dout, const float* lse, void* ws, int BH,
                          int N, int d, hipStream_t stream) {
  const WsLayout w = ws_layout(ws, BH, N);
  const int Npad = pad_rows(N);
  const size_t prow = (size_t)BH * Npad;
  const size_t threads = prow * (d / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  const uint16_t* o16 = (const uint16_t*)o;
  const uint16_t* g16 = (const uint16_t*)dout;
  if (d == 256)
    hipLaunchKernelGGL(bwd_pre_kernel<256>, dim3(blocks), dim3(256), 0, stream, o16, g16, lse,
                       w.l2, w.dv, (float*)nullptr, N, Npad, prow);
  else if (d == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(blocks), dim3(256), 0, stream, o16, g16, lse,
                       w.l2, w.dv, (float*)nullptr, N, Npad, prow);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(blocks), dim3(256), 0, stream, o16, g16, lse,
                       w.l2, w.dv, w.dq, N, Npad, prow);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const void* dout,
                           void* dk, void* dv, void* ws, int BH, int Nq, int Nk, int d, int group,
                           int hsplit, bool causal, float scale, hipStream_t stream) {
  if (Nk <= 0) return hipSuccess;   // no keys: no dK / dV rows, dQ stays 0
  const WsLayout w = ws_layout(ws, BH, Nq);
  float* part = hsplit > 1 ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                                      bwd_workspace_bytes(BH, Nq, d))
                           : nullptr;
  hipError_t e;
  if (d == 256)
    e = causal ? launch_main<256, true>(q, k, v, dout, w, dk, dv, part, BH, Nq, Nk, group, hsplit,
                                        scale, stream)
               : launch_main<256, false>(q, k, v, dout, w, dk, dv, part, BH, Nq, Nk, group,
                                         hsplit, scale, stream);
  else if (d == 128)
    e = causal ? launch_main<128, true>(q, k, v, dout, w, dk, dv, part, BH, Nq, Nk, group, hsplit,
                                        scale, stream)
               : launch_main<128, false>(q, k, v, dout, w, dk, dv, part, BH, Nq, Nk, group,
                                         hsplit, scale, stream);
  else
    e = causal ? launch_main<64, true>(q, k, v, dout, w, dk, dv, part, BH, Nq, Nk, group, hsplit,
                                       scale, stream)
               : launch_main<64, false>(q, k, v, dout, w, dk, dv, part, BH, Nq, Nk, group, hsplit,
                                        scale, stream);
  if (e != hipSuccess || hsplit <= 1) return e;
  const size_t n8 = (size_t)(BH / group) * Nk * d / 8;
  hipLaunchKernelGGL(bwd_kv_reduce_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                     stream, part, (uint16_t*)dk, (uint16_t*)dv, n8, hsplit);
  return hipGetLastError();
}

hipError_t launch_zero_bf16(void* a, void* b, size_t elems, hipStream_t stream) {
  // bf16 tensors of d = 64 or 128 per row: a multiple of 8 elements
  const size_t n8 = elems / 8;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_pair_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     (uint32_t*)a, (uint32_t*)b, n8);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
                     const WsLayout& w, int BH, int Nq, int Nk, int group, float scale,
                     hipStream_t stream) {
  using C = DqCfg<D>;
  auto kern = bwd_dq_direct_kernel<D, CAUSAL>;
  hipError_t e =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
  if (e != hipSuccess) return e;
  const int nqt = (Nq + C::QB - 1) / C::QB;
  hipLaunchKernelGGL(kern, dim3(BH * nqt), dim3(64 * C::WAVES), C::SMEM, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     (const uint16_t*)dout, w.l2, w.dv, (uint16_t*)dq, BH, Nq, Nk, Nk - Nq,
                     pad_rows(Nq), nqt, group, scale, scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_bwd_finalize(const void* q, const void* k, const void* v, const void* dout,
                               void* dq, const void* ws, int BH, int Nq, int Nk, int d, int group,
                               bool causal, float scale, hipStream_t stream) {
  const WsLayout w = ws_layout(const_cast<void*>(ws), BH, Nq);
  if (d == 64) {
    const size_t n8 = (size_t)BH * Nq * d / 8;
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                       w.dq, (uint16_t*)dq, n8);
    return hipGetLastError();
  }
  if (Nk <= 0) return launch_zero_bf16(dq, dq, (size_t)BH * Nq * d, stream);
  if (d == 256)
    return causal ? launch_dq<256, true>(q, k, v, dout, dq, w, BH, Nq, Nk, group, scale, stream)
                  : launch_dq<256, false>(q, k, v, dout, dq, w, BH, Nq, Nk, group, scale, stream);
  return causal ? launch_dq<128, true>(q, k, v, dout, dq, w, BH, Nq, Nk, group, scale, stream)
                : launch_dq<128, false>(q, k, v, dout, dq, w, BH, Nq, Nk, group, scale, stream);
}

}  // namespace fa
