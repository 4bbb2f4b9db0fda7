// Forward kernels: exact attention with online softmax, gfx950.
//
// One workgroup owns one tile of 128 queries of one (batch, head) and streams
// the key/value tiles past it (the flipped loop order of "Flash Attention,
// From First Principles", "The schedule -- who commutes?": the query block is
// resident, its output is written once).  Each of the 4 waves owns 32 query
// rows.  Per key tile a wave
//   1. mints the score tile on the matrix cores, transposed: S^T = K Q^T, so
//      each lane holds the scores of ONE query against 16 keys and its partner
//      lane (32 away) the other 16 ("The scaffold": S_tile = Q_tile K_tile^T);
//   2. masks keys past N and, on diagonal tiles, keys after the query;
//   3. takes the row max (in-lane, then one cross-half exchange) and updates
//      the running max m; rescales the running sum l and the accumulator by
//      exp(m_old - m_new) ("LLM Architecture Refresh [3]", sections 2 and 4);
//   4. forms P = exp(S - m_new) in fp32, adds its row sum to l, rounds P to
//      bf16 and accumulates O^T += V^T P^T on the matrix cores -- the bf16 P
//      registers are already in the B-operand layout, no data movement;
// and after the last tile divides once by l and stores O and the
// log-sum-exp ("FlashAttention from scratch", Step 3 and Follow-up questions).
// Key tiles lying wholly after a wave's last query are skipped
// ("LLM Architecture Refresh [3]", section 7).
//
// Scores are kept in log2 units: t = s * c - m with c = |scale| * log2(e), so
// each probability costs one FMA and one v_exp_f32.  A negative scale is
// handled by negating the query fragment (exact in bf16/fp32).
//
// K and V tiles go from HBM straight into LDS by DMA (global_load_lds), two
// stages deep: tile kt+1 is in flight while tile kt is computed, with one
// barrier per tile.  Both tiles stay row-major in LDS (XOR-swizzled against
// bank conflicts); the V^T operand of the PV product is read with the
// transposing ds_read_b64_tr_b16, so no register shuffling is needed.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // queries per workgroup

template <int D, int BN>
struct FwdCfg {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per tile row
  static constexpr int TILE_BYTES = BN * D * 2;     // one K or V tile (bf16)
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int SMEM_BYTES = 2 * STAGE_BYTES;
  static constexpr int NSB = BN / 32;               // 32-key sub-blocks per tile
  static constexpr int NKC = BN / 16;               // 16-key chunks per tile
  static constexpr int NQC = D / 16;                // 16-feature chunks (QK^T k-steps)
  static constexpr int NDB = D / 32;                // 32-feature output blocks
  static constexpr int DMA = TILE_BYTES / 16 / 256; // 16-byte DMAs per thread per tensor
  static constexpr int ROW_BYTES = CPR * 16;
  static_assert(DMA * 256 * 16 == TILE_BYTES, "tile split");
};

// Per-lane byte offset (inside one (batch, head) slice, relative to row k0) of
// the global chunk that lands in this lane's LDS slot of DMA number i.  Rows
// past N are clamped to row N-1 (finite data; those keys are masked to -inf
// and their P is 0, so they contribute nothing).
template <int D, int BN, int KIND>
__device__ __forceinline__ unsigned dma_src_off(int i, int w, int lane, int k0, int N, bool full) {
  using C = FwdCfg<D, BN>;
  const int slot = (i * 4 + w) * 64 + lane;
  const int row = slot / C::CPR;
  const int chunk = (slot % C::CPR) ^ swz<C::CPR, KIND>(row);
  const int src_row = full ? row : min(k0 + row, N - 1) - k0;
  return (unsigned)((src_row * D + chunk * 8) * 2);
}

template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int BH, int N, int nqt, float c, int negq) {
  using C = FwdCfg<D, BN>;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;

  int bh, qt;
  map_tile(blockIdx.x, BH, nqt, CAUSAL, &bh, &qt);
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + base;
  const char* Kb = reinterpret_cast<const char*>(K + base);
  const char* Vb = reinterpret_cast<const char*>(V + base);

  const int q0 = qt * kBM;
  const int wq0 = q0 + 32 * w;       // this wave's first query
  const int qrow = wq0 + n;          // this lane's query

  const int kend = CAUSAL ? min(N, q0 + kBM) : N;
  const int nkt = (kend + BN - 1) / BN;

  // DMA bookkeeping: LDS address of this wave's first 1 KiB slot, and the
  // per-lane source offsets of full tiles (K row-swizzled, V tr-swizzled).
  // DMA number i covers rows 16i*... further down the tile: with either
  // swizzle the lane's chunk does not depend on i, so one offset per tensor
  // plus a uniform stride of 4 KiB per DMA covers the tile.
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem_raw)) + w * 1024;
  const unsigned koff0 = dma_src_off<D, BN, SWZ_ROWS>(0, w, lane, 0, N, true);
  const unsigned voff0 = dma_src_off<D, BN, SWZ_TR>(0, w, lane, 0, N, true);
  auto issue = [&](int kt) {
    const int k0 = kt * BN;
    const char* kg = Kb + (size_t)k0 * D * 2;
    const char* vg = Vb + (size_t)k0 * D * 2;
    const unsigned st = lds0 + (kt & 1) * C::STAGE_BYTES;
    if (k0 + BN <= N) {
#pragma unroll
      for (int i = 0; i < C::DMA; ++i) {
        dma16(kg + i * 4096, koff0, st + i * 4096);
        dma16(vg + i * 4096, voff0, st + C::TILE_BYTES + i * 4096);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::DMA; ++i) {
        dma16(kg, dma_src_off<D, BN, SWZ_ROWS>(i, w, lane, k0, N, false), st + i * 4096);
        dma16(vg, dma_src_off<D, BN, SWZ_TR>(i, w, lane, k0, N, false),
              st + C::TILE_BYTES + i * 4096);
      }
    }
  };
  if (nkt > 0) issue(0);

  // Q^T as the B operand: lane holds Q[qrow][16c + 8h .. 16c + 8h + 7].
  bf16x8 qf[C::NQC];
  {
    const uint32_t flip = negq ? 0x80008000u : 0u;
#pragma unroll
    for (int cc = 0; cc < C::NQC; ++cc) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qrow < N) raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + 16 * cc + 8 * h);
      raw ^= flip;
      qf[cc] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // per-lane LDS operand offsets inside a stage.  K (A operand of S^T): row
  // 32sb + n, features 16cc + 8h..; the swizzle does not change with sb.
  int kb[C::NQC];
#pragma unroll
  for (int cc = 0; cc < C::NQC; ++cc) kb[cc] = tile_off<C::CPR, SWZ_ROWS>(n, 16 * cc + 8 * h);
  // V^T (A operand of O^T += V^T P^T) through transposing reads: 16-lane group
  // g reads key rows 4*(g/2) + j (+16kc, +8 for the second half) and features
  // 32db + 16*(g%2) + 4*(lane%4); the swizzle does not change with kc.
  const int vrow0 = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int vcol0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int vb[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) vb[db] = tile_off<C::CPR, SWZ_TR>(vrow0, 32 * db + vcol0);

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kNegInf;   // running max, log2-scaled units
  float lsum = 0.f;    // this lane's share of the running sum

  const char* smem_k = smem_raw;
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BN;
    // tile kt has landed for every lane; every wave is done with tile kt-1
    wait_vmem();
    __syncthreads();
    if (kt + 1 < nkt) issue(kt + 1);
    const char* ks = smem_k + (kt & 1) * C::STAGE_BYTES;
    const char* vs = ks + C::TILE_BYTES;

    // sub-blocks of 32 keys this wave must compute (wave-uniform)
    int nsb = C::NSB;
    if (CAUSAL) {
      const int lim = wq0 + 31 - k0;          // last visible key offset for the wave
      nsb = lim < 0 ? 0 : min(C::NSB, lim / 32 + 1);
    }
    if (nsb == 0) continue;

    f32x16 s[C::NSB];
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
      if (sb < nsb) {
        bf16x8 a[C::NQC];
#pragma unroll
        for (int cc = 0; cc < C::NQC; ++cc)
          a[cc] = *reinterpret_cast<const bf16x8*>(ks + kb[cc] + sb * 32 * C::ROW_BYTES);
        const f32x16 zero = {};
        s[sb] = mfma_32x32x16_bf16(a[0], qf[0], zero);
#pragma unroll
        for (int cc = 1; cc < C::NQC; ++cc) s[sb] = mfma_32x32x16_bf16(a[cc], qf[cc], s[sb]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sb][r] = kNegInf;
      }
    }

    // mask: register r of sub-block sb holds key k0 + 4h + off(sb, r) with
    // off = 32sb + 8(r/4) + r%4; it is dead past the lane's limit (its own
    // query under causal masking, and N - 1)
    if ((k0 + BN > N) || (CAUSAL && k0 + BN - 1 > wq0)) {
      int lim = N - 1 - k0 - 4 * h;
      if (CAUSAL) lim = min(lim, qrow - k0 - 4 * h);
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * sb + 8 * (r >> 2) + (r & 3);
          s[sb][r] = off > lim ? kNegInf : s[sb][r];
        }
    }

    float mx = kNegInf;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m, mx * c);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);

    // P = exp2(s*c - m), summed in fp32 (the saved lse needs the unrounded
    // sum: rounding each p to bf16 first moves ln(l) by up to 2^-9 on short
    // rows), then rounded to bf16 for the PV product
    uint32_t pk[C::NSB][8];
    float ps = 0.f;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], c, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r + 1], c, -m_use));
        pk[sb][r >> 1] = pack_bf16x2(p0, p1);
        ps += p0 + p1;
      }
    lsum = lsum * alpha + ps;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
    m = m_new;

    // O^T += V^T P^T over the computed sub-blocks
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
      if (sb < nsb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kc = 2 * sb + half;
          const bf16x8 b = __builtin_bit_cast(
              bf16x8, u32x4{pk[sb][4 * half + 0], pk[sb][4 * half + 1], pk[sb][4 * half + 2],
                            pk[sb][4 * half + 3]});
          bf16x8 a[C::NDB];
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const u32x2 lo = lds_read_tr16(vs + vb[db] + (16 * kc) * C::ROW_BYTES);
            const u32x2 hi = lds_read_tr16(vs + vb[db] + (16 * kc + 8) * C::ROW_BYTES);
            a[db] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
          }
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) acc[db] = mfma_32x32x16_bf16(a[db], b, acc[db]);
        }
      }
    }
  }

  // epilogue: one deferred division, then O and the log-sum-exp
  const float lt = lsum + wave_xor32(lsum);
  const float inv = 1.f / lt;
  if (qrow < N) {
    uint16_t* orow = O + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        u32x2 out = {pack_bf16x2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                     pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = out;
      }
    if (h == 0) LSE[(size_t)bh * N + qrow] = (m + __log2f(lt)) * kLn2;
  }
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
  const int q0 = qt * kBM;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + n;

  // B operand of S^T = K Q^T: lane holds Q[qrow][2i + h]
  float qf[D / 2];
#pragma unroll
  for (int i = 0; i < D / 2; ++i) {
    float x = (qrow < N) ? Qh[(size_t)qrow * D + 2 * i + h] : 0.f;
    qf[i] = negq ? -x : x;
  }

  const int kend = CAUSAL ? min(N, q0 + kBM) : N;
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

// Softmax scale in log2 units.  scale == 0 (uniform attention) uses a tiny
// positive factor instead so masked scores still map to -inf, never NaN:
// every finite score then rounds to the same exponent, 0.
inline void split_scale(float scale, float* c, int* negq) {
  *negq = scale < 0.f;
  float a = scale < 0.f ? -scale : scale;
  *c = a > 0.f ? a * kLog2e : 1e-30f;
}

template <int D, int BN, bool CAUSAL>
hipError_t launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                       int N, float scale, hipStream_t stream) {
  using C = FwdCfg<D, BN>;
  const int nqt = (N + kBM - 1) / kBM;
  float c;
  int negq;
  split_scale(scale, &c, &negq);
  auto kern = fwd_bf16_kernel<D, BN, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(BH * nqt), dim3(256), C::SMEM_BYTES, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                     BH, N, nqt, c, negq);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                      int BH, int N, float scale, hipStream_t stream) {
  using C = FwdF32Cfg<D>;
  const int nqt = (N + kBM - 1) / kBM;
  float c;
  int negq;
  split_scale(scale, &c, &negq);
  auto kern = fwd_f32_kernel<D, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(BH * nqt), dim3(256), C::SMEM_BYTES, stream, q, k, v, o, lse, BH,
                     N, nqt, c, negq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int BH, int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_bf16<128, 64, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_bf16<128, 64, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch_bf16<64, 128, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_bf16<64, 128, false>(q, k, v, o, lse, BH, N, scale, stream);
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
