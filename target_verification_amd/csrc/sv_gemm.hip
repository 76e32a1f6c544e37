// Dequant-fused GEMM on the matrix cores: for each group of 16*TPW output
// columns, y[m][c] = sum over k of x[m][k] * w[c][k], computed as K-split
// partials that are summed in a fixed order and then passed through the
// fused epilogue.
//
// Two kernels compute identical bits for every row:
//  * k_qgemm (up to 32 rows per launch): one workgroup per column group, one
//    wave per K split; the splits meet in LDS and the workgroup applies the
//    group's epilogue.
//  * k_qgemm_wide (more rows, when the tensor has enough column sets to keep
//    the CUs busy; otherwise k_qgemm runs once per pair of M-tiles): one
//    wave per (64 columns, up to 48 rows) walks
//    the tensor's K splits in turn, keeping each split's partial apart from
//    the running sum, so the summation order is the same as above; it then
//    applies the epilogue to its own rows.
//
// A wave streams the tile-blocks of its column tiles (16 B per lane per
// load, fully coalesced), turns the integer codes into exact fp16 operands
// in registers, and issues v_mfma_f32_16x16x32_f16 with the activation's fp16
// high part and its low part (scaled by 2^11) against the weight operand,
// into two accumulators joined once per super-block as hi + 2^-11 lo.  A
// launch whose M-tile holds at most 8 rows puts the high parts in MFMA rows
// 0..7 and the low parts in rows 8..15 of one operand instead, so a single
// product per k-step yields both (each MFMA row is its own dot product: the
// bits are those of the two separate products).
//
// Scales: the 6-bit sub-block scale of the 4-bit super-block format is an
// exact integer factor folded into the fp16 operand (sc * q <= 945); the
// 6-bit format's sc * (q - 32) is split into an exact fp16 high part and a
// remainder in {-1, 0, 1}; the super scale d is applied in fp32 once per
// super-block.  The 4-bit super-block's min term sum_j m_j Sx_j is a small
// product of the packed sub-block sums Sx with the exact integers m_j, scaled
// by dmin in fp32.  The 4-bit/32 format applies its block scale per k-step.
//
// Load order: k_qgemm refills each k-step's activation registers with the
// next super-block's as soon as that k-step's products are issued, and keeps
// two weight buffers (super-block sb + 2 is requested when sb is done); for
// the 4-bit formats one load brings the records of all of a wave's tiles,
// and for at most 4 packed rows one load brings two k-steps of activations;
// k_qgemm_wide keeps DA k-steps of activations and three super-blocks of
// weights in flight.  Loads complete in issue order, so each wait covers
// only loads issued about a step earlier.  Direct global -> LDS loads are
// issued only after the main loops: issued before them, they make the
// compiler wait for every outstanding load at each step.
//
// The result of a row depends only on that row's activations and on the
// fixed K split of the tensor, never on how many rows the call carries or
// which kernel runs it.

#include "sv_gemm_body.h"

template <int FMT, int TPW, int MTP, int EPI>
__global__ __launch_bounds__(64 * SV_MAX_KSPLIT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_qgemm(const uint8_t *__restrict__ W, int nsb, int ksplit, int sbps,
             const uint8_t *__restrict__ ap, const uint8_t *__restrict__ sx, int M, int mt0,
             int MTall, sv_epi_args ea) {
  __shared__ float s_inv[64];
  extern __shared__ __attribute__((aligned(16))) float s_dyn[];
#ifdef SV_TIMELINE
  const long long t0 = sv_tl_now();
#endif
  // workgroup = column group, wave = K split
  qgemm_body<FMT, TPW, MTP, EPI, false, false>(W, nsb, ksplit, sbps, ap, sx, M, mt0, MTall, ea,
                                        blockIdx.x, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6),
                                        true, threadIdx.x, blockDim.x, s_dyn, s_inv, [] {});
#ifdef SV_TIMELINE
  if (threadIdx.x == 0) {
    sv_tl_put(ea.layer, ea.tl_kind, blockIdx.x, SV_TLF_EPI, sv_tl_now());
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    sv_tl_put(ea.layer, ea.tl_kind, blockIdx.x, SV_TLF_STORED, sv_tl_now());
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    sv_tl_put(ea.layer, ea.tl_kind, blockIdx.x, SV_TLF_START, t0);
    sv_tl_put(ea.layer, ea.tl_kind, blockIdx.x, SV_TLF_END, sv_tl_now());
  }
#endif
}
// ---- wide-M kernel -----------------------------------------------------------
// Workgroup: 4 waves on the same 4 column tiles (64 columns), each wave with
// MWW M-tiles of its own.  Per super-block, every wave multiplies its rows
// against all four tiles of one LDS stage (their operands read one k-step
// ahead, its activation operands streamed from L2 four k-steps ahead) while
// turning the codes of tile w, k-step by k-step, into the fp16 operands of
// the next super-block in the other stage (double-buffered, one barrier per
// super-block).  Blocks are
// dealt to the 8 XCDs in turn; the logical block index keeps consecutive
// logical blocks (the M groups of one column set, which read the same
// weights) on one XCD so that they share its L2.
#define SV_WIDE_CT 4

template <int FMT>
struct wide_stage {
  static constexpr int KB = (FMT == SV_B6_256) ? 2 : 1;          // operands per (tile, k-step)
  static constexpr int OPS = SV_WIDE_CT * 8 * KB * 1024;         // weight operands
  static constexpr int MINS = (FMT == SV_B4_256) ? SV_WIDE_CT * 1024 : 0;   // min operands
  static constexpr int NSC = (FMT == SV_B4_32) ? 8 : (FMT == SV_B4_256 ? 2 : 1);
  static constexpr int SCALES = SV_WIDE_CT * 16 * NSC * 4;       // fp32 scales per column
  static constexpr int BYTES = OPS + MINS + SCALES;
};

template <int FMT, int MWW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_qgemm_wide(const uint8_t *__restrict__ W, int nsb, int sbps,
                  const uint8_t *__restrict__ ap, const uint8_t *__restrict__ sx, int M, int mt0,
                  int mtend, int MTall, int mgroups, sv_epi_args ea) {
  constexpr int CT = SV_WIDE_CT, C4 = 16 * CT, MLOC = 16 * MWW;
  constexpr int DA = 4;   // activation k-steps in flight (a ring indexed by k-step % DA)
  static_assert(8 % DA == 0, "the activation ring must tile a super-block's 8 k-steps");
  typedef wide_stage<FMT> ST;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
  const int nblk = gridDim.x, b = blockIdx.x, full = nblk & ~7;
  const int L = b < full ? (b & 7) * (full >> 3) + (b >> 3) : b;
  const int cs = L / mgroups, mgi = L - cs * mgroups;
  const int mtw = mt0 + (mgi * 4 + wv) * MWW;   // this wave's first M-tile
  const bool rows = mtw < mtend;                 // (a wave without rows still
                                                 // makes its tile's operands)
  const int KS = nsb * 8;
  constexpr int TB = (FMT == SV_B6_256) ? SV_TB_B6 : SV_TB_B4;
  constexpr int NC = (FMT == SV_B6_256) ? 3 : 2;
  constexpr uint32_t kOOB = 0x80000000u;   // past the resource: zeros, no traffic
  const uint32_t mg = vconst(0x64006400u), mg64 = vconst(0x54005400u);
  // this wave's tile of the column set
  const rsrc_t wr = make_rsrc(W + ((size_t)cs * CT + wv) * nsb * TB, (uint32_t)(nsb * TB));
  const rsrc_t ar = make_rsrc(ap, (uint32_t)(MTall * KS * 2048));
  const rsrc_t sr = make_rsrc(sx, (uint32_t)(MTall * nsb * 512));

  extern __shared__ __attribute__((aligned(16))) uint8_t s_raw[];

  // M-tiles past the launch's range load zeros; padding rows of a tile read
  // row 0 of their lane group (outputs never stored)
  uint32_t alane[MWW], aoob[MWW];
  int mtc[MWW];
#pragma unroll
  for (int i = 0; i < MWW; ++i) {
    const int mt = mtw + i;
    const bool in = mt < mtend;
    mtc[i] = in ? mt : mt0;
    aoob[i] = in ? 0u : kOOB;
    alane[i] = 16u * (uint32_t)apack_piece((16 * mt + n16 < M) ? n16 : 0, g, M);
  }

  u32x4 rec[2], cod[2][NC];
  uint32_t dd[2];
  auto load_w = [&](int sb, int buf) {
    const uint32_t oob = sb < nsb ? 0u : kOOB;
    const uint32_t tb = (uint32_t)((sb < nsb ? sb : 0) * TB) | oob;
    rec[buf] = bload16(wr, tb + 16 * n16);
    if (FMT == SV_B6_256) {
      dd[buf] = bload2(wr, tb + 256 + 2 * n16);
      cod[buf][0] = bload16(wr, tb + 288 + 16 * lane);
      cod[buf][1] = bload16(wr, tb + 288 + 1024 + 16 * lane);
      cod[buf][2] = bload16(wr, tb + 2336 + 16 * lane);
    } else {
      dd[buf] = 0;
      cod[buf][0] = bload16(wr, tb + 256 + 16 * lane);
      cod[buf][1] = bload16(wr, tb + 256 + 1024 + 16 * lane);
    }
  };
  half8 Ah[DA][MWW], Al[DA][MWW];
  auto load_a = [&](int p, int slot) {   // p = 8 * super-block + k-step
    const uint32_t oob = p < KS ? 0u : kOOB;
    const int pc = p < KS ? p : 0;
#pragma unroll
    for (int i = 0; i < MWW; ++i) {
      const uint32_t base = (uint32_t)((mtc[i] * KS + pc) * 2048) | oob | aoob[i];
      Ah[slot][i] = make_half8(bload16(ar, base + alane[i]));
      Al[slot][i] = make_half8(bload16(ar, base + 1024 + alane[i]));
    }
  };
  half8 shi[MWW], slo[MWW];
  auto load_s = [&](int sb) {
    if (FMT != SV_B4_256) return;
    const uint32_t oob = sb < nsb ? 0u : kOOB;
    const int sbc = sb < nsb ? sb : 0;
#pragma unroll
    for (int i = 0; i < MWW; ++i) {
      const int row = (16 * (mtw + i) + n16 < M) ? n16 : 0;
      // lane groups 1..3 (k slots 8..31 of the min product) read zeros
      const uint32_t gz = g == 0 ? 0u : kOOB;
      shi[i] = make_half8(bload16(sr, (uint32_t)sxpack_off(mtc[i], nsb, sbc, 0, row) | oob | aoob[i] | gz));
      slo[i] = make_half8(bload16(sr, (uint32_t)sxpack_off(mtc[i], nsb, sbc, 1, row) | oob | aoob[i] | gz));
    }
  };

  // LDS stage: operands [tile][k-step][part][lane] (16 B each), then the
  // min operands [tile][lane], then fp32 scales [tile][slot][column]
  auto st_ops = [&](int buf) { return (half8 *)(s_raw + buf * ST::BYTES); };
  auto st_mins = [&](int buf) { return (half8 *)(s_raw + buf * ST::BYTES + ST::OPS); };
  auto st_sc = [&](int buf) { return (float *)(s_raw + buf * ST::BYTES + ST::OPS + ST::MINS); };

  // this wave's tile of a super-block (weights in register buffer buf) into
  // LDS stage buf: k-step ks, then the super-block's mins and scales
  auto produce_ks = [&](int buf, int ks) {
    const u32x4 r = rec[buf];
    half8 *ops = st_ops(buf) + (size_t)wv * 8 * ST::KB * 64;
    float *sc = st_sc(buf) + wv * 16 * ST::NSC;
    {
      if (FMT == SV_B4_256) {
        ops[ks * 64 + lane] = b4s_op(r, cod[buf][ks >> 2][ks & 3], ks, mg, mg64);
      } else if (FMT == SV_B4_32) {
        ops[ks * 64 + lane] = b432_op(cod[buf][ks >> 2][ks & 3], mg, mg64);
        if (lane < 16) sc[ks * 16 + n16] = f16_at(r[ks >> 1], ks & 1);
      } else {
        half8 bhi, blo;
        b6_op(cod[buf], r, ks, g, mg, bhi, blo);
        ops[(2 * ks) * 64 + lane] = bhi;
        ops[(2 * ks + 1) * 64 + lane] = blo;
      }
    }
  };
  auto produce_sb = [&](int buf) {
    const u32x4 r = rec[buf];
    float *sc = st_sc(buf) + wv * 16 * ST::NSC;
    if (FMT == SV_B4_256) {
      st_mins(buf)[wv * 64 + lane] = b4s_min_op(r, mg);
      if (lane < 16) {
        sc[n16] = f16_at(r[0], 0);
        sc[16 + n16] = f16_at(r[0], 1);
      }
    } else if (FMT == SV_B6_256) {
      if (lane < 16) sc[n16] = f16_at(dd[buf], 0);
    }
  };
  auto produce = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) produce_ks(buf, ks);
    produce_sb(buf);
  };

  floatx4 P[CT][MWW], tot[CT][MWW];
#pragma unroll
  for (int t = 0; t < CT; ++t)
#pragma unroll
    for (int i = 0; i < MWW; ++i) P[t][i] = tot[t][i] = floatx4{0.f, 0.f, 0.f, 0.f};

  // this wave's rows against the four tiles of super-block sb (LDS stage buf)
  // The next super-block's operands are made k-step by k-step between this
  // super-block's products (their VALU work then overlaps the matrix cores;
  // batch-12 block round 5.04 -> 4.92 ms), except for the 4-bit/32 format,
  // whose kernels would spill at that register pressure.
  constexpr bool ILV = FMT != SV_B4_32;
  // pbuf: the stage to make the next super-block's operands in (or -1)
  auto consume = [&](int sb, int buf, int pbuf) {
    const half8 *ops = st_ops(buf);
    const float *sc = st_sc(buf);
    floatx4 Th[CT][MWW], Tl[CT][MWW];
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int i = 0; i < MWW; ++i) Th[t][i] = Tl[t][i] = floatx4{0.f, 0.f, 0.f, 0.f};
    // The stage's operands of every tile for k-step ks are read from LDS
    // one k-step ahead into two alternating register sets: read just before
    // their products (as the compiler schedules them under this register
    // pressure), each wait on LDS stalled the wave's matrix cores (batch-12
    // block round 5.33 -> 5.12 ms).
    constexpr int KB = ST::KB;
    half8 bq[2][CT][KB];
    auto ldb = [&](int ks, int set) {
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) bq[set][t][kb] = ops[((t * 8 + ks) * KB + kb) * 64 + lane];
    };
    ldb(0, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int slot = ks % DA;
      if (ks + 1 < 8) ldb(ks + 1, (ks + 1) & 1);
      if (ILV && pbuf >= 0) produce_ks(pbuf, ks);
      __builtin_amdgcn_sched_barrier(0);
      auto bop = [&](int t, int kb) { return bq[ks & 1][t][kb]; };
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        if (FMT == SV_B4_256) {
          const half8 bw = bop(t, 0);
#pragma unroll
          for (int i = 0; i < MWW; ++i) {
            Th[t][i] = mfma16(Ah[slot][i], bw, Th[t][i]);
            Tl[t][i] = mfma16(Al[slot][i], bw, Tl[t][i]);
          }
        } else if (FMT == SV_B4_32) {
          const half8 bw = bop(t, 0);
          const float d = sc[(t * 8 + ks) * 16 + n16];
#pragma unroll
          for (int i = 0; i < MWW; ++i) {
            const floatx4 z0 = {0.f, 0.f, 0.f, 0.f};
            P[t][i] = upd_d(P[t][i], mfma16(Ah[slot][i], bw, z0), mfma16(Al[slot][i], bw, z0), d);
          }
        } else {
          const half8 bhi = bop(t, 0);
          const half8 blo = bop(t, KB - 1);
#pragma unroll
          for (int i = 0; i < MWW; ++i) {
            Th[t][i] = mfma16(Ah[slot][i], bhi, Th[t][i]);
            Th[t][i] = mfma16(Ah[slot][i], blo, Th[t][i]);
            Tl[t][i] = mfma16(Al[slot][i], bhi, Tl[t][i]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_a(8 * sb + ks + DA, slot);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (FMT == SV_B4_256) {
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        const half8 bm = st_mins(buf)[t * 64 + lane];
        const float d = sc[t * 32 + n16], dmin = sc[t * 32 + 16 + n16];
#pragma unroll
        for (int i = 0; i < MWW; ++i) {
          const floatx4 z0 = {0.f, 0.f, 0.f, 0.f};
          const floatx4 uh = mfma16(shi[i], bm, z0);
          const floatx4 ul = mfma16(slo[i], bm, z0);
          P[t][i] = upd_b4s(P[t][i], Th[t][i], Tl[t][i], uh, ul, d, dmin);
        }
      }
    } else if (FMT == SV_B6_256) {
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        const float d = sc[t * 16 + n16];
#pragma unroll
        for (int i = 0; i < MWW; ++i) P[t][i] = upd_d(P[t][i], Th[t][i], Tl[t][i], d);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_s(sb + 1);
    __builtin_amdgcn_sched_barrier(0);
    // end of a K split: add its partial to the running sum (in split order)
    if ((sb + 1) % sbps == 0 || sb + 1 == nsb) {
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int i = 0; i < MWW; ++i) {
          tot[t][i] = tot[t][i] + P[t][i];
          P[t][i] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
  };
  // LDS writes of this wave done, then every wave of the workgroup (global
  // loads stay in flight across it)
  auto stage_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // Iteration sb: multiply super-block sb (stage sb & 1) while making the
  // operands of super-block sb + 1 (register buffer and stage (sb + 1) & 1),
  // refill that register buffer with super-block sb + 3, barrier.
  load_w(0, 0);
#pragma unroll
  for (int j = 0; j < DA; ++j) load_a(j, j);
  load_s(0);
  load_w(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  produce(0);
  __builtin_amdgcn_sched_barrier(0);
  load_w(2, 0);
  stage_barrier();
  auto iter = [&](int sb, int cur) {
    const int nxt = cur ^ 1;
    if constexpr (ILV) {
      // the next super-block's operands between this one's products, then
      // its register buffer is refilled
      consume(sb, cur, sb + 1 < nsb ? nxt : -1);
      if (sb + 1 < nsb) produce_sb(nxt);
      __builtin_amdgcn_sched_barrier(0);
      load_w(sb + 3, nxt);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      if (sb + 1 < nsb) produce(nxt);
      __builtin_amdgcn_sched_barrier(0);
      load_w(sb + 3, nxt);
      __builtin_amdgcn_sched_barrier(0);
      consume(sb, cur, -1);
    }
    stage_barrier();
  };
  int sb = 0;
  for (; sb + 1 < nsb; sb += 2) {
    iter(sb, 0);
    iter(sb + 1, 1);
  }
  if (sb < nsb) iter(sb, 0);

  if (!rows) return;
  // this wave's sums to LDS (the stages are free after the last barrier) as
  // [group][MLOC][C], then the group epilogues
  const int m0 = 16 * mtw, m1 = min(M, 16 * min(mtw + MWW, mtend));
  float *const s_tot = (float *)s_raw + (size_t)wv * (MLOC * C4 + MLOC);
  float *const s_inv = s_tot + MLOC * C4;
  const int C = ea.C, gpw = C4 / C;
#pragma unroll
  for (int t = 0; t < CT; ++t)
#pragma unroll
    for (int i = 0; i < MWW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cw = 16 * t + n16, gl = cw / C, col = cw - gl * C;
        s_tot[(gl * MLOC + 16 * i + 4 * g + r) * C + col] = tot[t][i][r];
      }
  if (lane < m1 - m0) s_inv[lane] = ea.rowscale ? ea.rowscale[m0 + lane] : 1.0f;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // one wave writes and reads
  for (int gl = 0; gl < gpw; ++gl)
    sv_epi::epi_rows(ea, cs * gpw + gl, m0, m1, lane, 64, s_inv, s_tot + gl * MLOC * C, MLOC, 1);
}

template <int FMT, int MWW>
static constexpr size_t wide_lds_bytes() {
  return (2 * (size_t)wide_stage<FMT>::BYTES > sizeof(float) * 4 * (16 * MWW * 16 * SV_WIDE_CT + 16 * MWW))
             ? 2 * (size_t)wide_stage<FMT>::BYTES
             : sizeof(float) * 4 * (16 * MWW * 16 * SV_WIDE_CT + 16 * MWW);
}

// Row norm factors of all M rows into rinv (one wave per row; the same
// reduction as the small-M kernel's LDS path).
__global__ __launch_bounds__(256) void k_rowscale(sv_epi_args ea, float *rinv) {
  const int m = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (m >= ea.M) return;
  sv_epi::row_scales_lds(ea, m, m + 1, threadIdx.x & 63, ea.ssq + (size_t)m * ea.nssq, rinv + m);
}

size_t sv_gemm_lds_bytes(int ksplit, int MT, int TPW, const sv_epi_args &ea) {
  return sizeof(float) * ((size_t)ksplit * 16 * MT * 16 * TPW + (ea.ssq ? 16 * MT * ea.nssq : 0) +
                          (ea.type == SV_EPI_RESID ? 16 * MT * 32 + 32 : 0) +
                          (ea.type == SV_EPI_RESID || ea.type == SV_EPI_SWIGLU ? 16 * MT * 64 : 0));
}

template <int FMT, int TPW, int MTP, int EPI>
static hipError_t allow_lds() {
  return hipFuncSetAttribute((const void *)k_qgemm<FMT, TPW, MTP, EPI>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, 140 * 1024);
}

template <int FMT, int MWW>
static hipError_t allow_lds_wide() {
  return hipFuncSetAttribute((const void *)k_qgemm_wide<FMT, MWW>,
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)wide_lds_bytes<FMT, MWW>());
}

// Raise the dynamic LDS limit of every GEMM instantiation (host call made at
// model or weight creation, never inside a round).
hipError_t sv_gemm_prepare() {
  static bool done = false;
  if (done) return hipSuccess;
  hipError_t e = hipSuccess;
#define SV_ALLOW(F, T, E)                                         \
  if (e == hipSuccess) e = allow_lds<F, T, 1, E>();               \
  if constexpr (T < 4) {                                          \
    if (e == hipSuccess) e = allow_lds<F, T, 2, E>();             \
  }                                                               \
  if constexpr (F == SV_B4_256 || F == SV_B6_256) {              \
    if (e == hipSuccess) e = allow_lds<F, T, SV_MT_PACK8, E>();   \
  }                                                               \
  if constexpr (F == SV_B4_256) {                                 \
    if (e == hipSuccess) e = allow_lds<F, T, SV_MT_PACK4, E>();   \
  }
  SV_ALLOW(SV_B4_256, 4, SV_EPI_ANY) SV_ALLOW(SV_B4_256, 2, SV_EPI_ANY)
  SV_ALLOW(SV_B4_32, 4, SV_EPI_ANY) SV_ALLOW(SV_B4_32, 2, SV_EPI_ANY)
  SV_ALLOW(SV_B6_256, 2, SV_EPI_ANY) SV_ALLOW(SV_B4_256, 2, SV_EPI_QKV)
  SV_ALLOW(SV_B4_256, 2, SV_EPI_RESID) SV_ALLOW(SV_B4_256, 4, SV_EPI_SWIGLU)
  SV_ALLOW(SV_B6_256, 2, SV_EPI_LM)
#undef SV_ALLOW
#define SV_ALLOW_WIDE(F)                                             \
  if (e == hipSuccess) e = allow_lds_wide<F, 1>();                 \
  if (e == hipSuccess) e = allow_lds_wide<F, 2>();                 \
  if (e == hipSuccess) e = allow_lds_wide<F, 3>();
  SV_ALLOW_WIDE(SV_B4_256) SV_ALLOW_WIDE(SV_B4_32) SV_ALLOW_WIDE(SV_B6_256)
#undef SV_ALLOW_WIDE
  done = (e == hipSuccess);
  return e;
}

template <int FMT, int TPW, int EPI>
static hipError_t launch_mt(const sv_qweight *w, const uint8_t *ap, const uint8_t *sx, int M,
                            int mt0, int mtn, const sv_epi_args &ea, hipStream_t st) {
  if (w->ksplit > SV_MAX_KSPLIT || ea.ksplit != w->ksplit || ea.C != 16 * TPW)
    return hipErrorInvalidValue;
  dim3 grid(w->ngroups), block(64 * w->ksplit);
  const int MTall = (M + 15) / 16;
  while (mtn > 0) {
    // at most 2 M-tiles per launch, 1 with four tiles per wave (two would
    // not fit the registers: the spilled variant ran 2.5x slower than two
    // one-tile launches, which stream the weights twice)
    const int n = (TPW < 4 && mtn >= 2) ? 2 : 1;
    // one M-tile of at most 8 rows: high and low parts share each product
    // (4-bit/256, at most 4 rows: two k-steps per activation load)
    const bool packed = (FMT == SV_B4_256 || FMT == SV_B6_256) && n == 1 && M - 16 * mt0 <= 8;
    const bool packed4 = FMT == SV_B4_256 && packed && M <= SV_APACK4_ROWS;
#define SV_GEMM_LAUNCH(N)                                                                     \
    hipLaunchKernelGGL((k_qgemm<FMT, TPW, N, EPI>), grid, block,                              \
                       sv_gemm_lds_bytes(w->ksplit, (N) == 1 || (N) == 2 ? (N) : 1, TPW, ea), \
                       st, w->data, w->nsb, w->ksplit, w->sbps, ap, sx, M, mt0, MTall, ea)
    if constexpr (FMT == SV_B4_256 && TPW < 4) {
      if (packed4) SV_GEMM_LAUNCH(SV_MT_PACK4);
      else if (packed) SV_GEMM_LAUNCH(SV_MT_PACK8);
      else if (n == 2) SV_GEMM_LAUNCH(2);
      else SV_GEMM_LAUNCH(1);
    } else if constexpr (FMT == SV_B4_256) {
      if (packed4) SV_GEMM_LAUNCH(SV_MT_PACK4);
      else if (packed) SV_GEMM_LAUNCH(SV_MT_PACK8);
      else SV_GEMM_LAUNCH(1);
    } else if constexpr (FMT == SV_B6_256 && TPW < 4) {
      if (packed) SV_GEMM_LAUNCH(SV_MT_PACK8);
      else if (n == 2) SV_GEMM_LAUNCH(2);
      else SV_GEMM_LAUNCH(1);
    } else if constexpr (FMT == SV_B6_256) {
      if (packed) SV_GEMM_LAUNCH(SV_MT_PACK8);
      else SV_GEMM_LAUNCH(1);
    } else if constexpr (TPW < 4) {
      if (n == 2) SV_GEMM_LAUNCH(2);
      else SV_GEMM_LAUNCH(1);
    } else {
      SV_GEMM_LAUNCH(1);
    }
#undef SV_GEMM_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    mt0 += n;
    mtn -= n;
  }
  return hipSuccess;
}

template <int FMT, int MWW>
static hipError_t launch_wide_mww(const sv_qweight *w, const uint8_t *ap, const uint8_t *sx,
                                  int M, int mt0, int mtn, const sv_epi_args &ea,
                                  hipStream_t st) {
  const int ncs = w->ntile / SV_WIDE_CT;
  const int mgroups = (mtn + 4 * MWW - 1) / (4 * MWW);
  const int MTall = (M + 15) / 16;
  const size_t lds = wide_lds_bytes<FMT, MWW>();
  hipLaunchKernelGGL((k_qgemm_wide<FMT, MWW>), dim3(ncs * mgroups), dim3(256), lds, st,
                     w->data, w->nsb, w->sbps, ap, sx, M, mt0, mt0 + mtn, MTall, mgroups, ea);
  return hipGetLastError();
}

// M-tiles per wave of the wide kernel: the rows spread over the 4 waves
// (at most 3 M-tiles each), fewer when that leaves under ~200 workgroups
// (fewer than most of the 256 CUs busy).
static int wide_mww(int ncs, int mtn) {
  int mww = (mtn + 3) / 4;
  if (mww > 3) mww = 3;
  if (mww < 1) mww = 1;
  while (mww > 1 && (long)ncs * ((mtn + 4 * mww - 1) / (4 * mww)) < 200) --mww;
  return mww;
}

template <int FMT>
static hipError_t launch_wide(const sv_qweight *w, const uint8_t *ap, const uint8_t *sx, int M,
                              int mt0, int mtn, const sv_epi_args &ea, hipStream_t st) {
  sv_epi_args e = ea;
  if (ea.ssq) {   // the row norm factors first, into rinv
    if (!ea.rinv) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_rowscale, dim3((M + 3) / 4), dim3(256), 0, st, ea, ea.rinv);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    e.rowscale = ea.rinv;
    e.ssq = nullptr;
  }
  int mww = wide_mww(w->ntile / SV_WIDE_CT, mtn);
  if (FMT == SV_B4_32) mww = 1;   // more M-tiles per wave would spill here
  switch (mww) {
    case 3: return launch_wide_mww<FMT, 3>(w, ap, sx, M, mt0, mtn, e, st);
    case 2: return launch_wide_mww<FMT, 2>(w, ap, sx, M, mt0, mtn, e, st);
    default: return launch_wide_mww<FMT, 1>(w, ap, sx, M, mt0, mtn, e, st);
  }
}

// More than two M-tiles go to the wide kernel (one launch) when it has
// work for most of the CUs even at one M-tile per wave (about 200
// workgroups); otherwise the small kernel runs once per one or two M-tiles
// (measured at 36-60 rows: o and down, 80 column sets, ran 1.6-2x faster
// that way).  The tensor must have whole 64-column sets and groups of at
// most 64 columns.  Both kernels give a row the same bits.
static bool use_wide(const sv_qweight *w, int mtn, const sv_epi_args &ea) {
  return mtn > 2 && w->ntile % SV_WIDE_CT == 0 && (16 * SV_WIDE_CT) % ea.C == 0 &&
         (long)(w->ntile / SV_WIDE_CT) * ((mtn + 3) / 4) >= 200;
}

hipError_t sv_launch_qgemm(const sv_qweight *w, const uint8_t *ap, const uint8_t *sx, int M,
                           int mt0, int mtn, const sv_epi_args &ea, hipStream_t st) {
  if (use_wide(w, mtn, ea)) {
    if (ea.ksplit != w->ksplit || ea.C != 16 * w->tpw) return hipErrorInvalidValue;
    if (w->type == SV_B4_256) return launch_wide<SV_B4_256>(w, ap, sx, M, mt0, mtn, ea, st);
    if (w->type == SV_B4_32) return launch_wide<SV_B4_32>(w, ap, sx, M, mt0, mtn, ea, st);
    return launch_wide<SV_B6_256>(w, ap, sx, M, mt0, mtn, ea, st);
  }
  // the round's own combinations run kernels specialised for their
  // epilogue; the rest read the epilogue type from the arguments
  if (w->type == SV_B4_256) {
    if (w->tpw == 4) {
      if (ea.type == SV_EPI_SWIGLU)
        return launch_mt<SV_B4_256, 4, SV_EPI_SWIGLU>(w, ap, sx, M, mt0, mtn, ea, st);
      return launch_mt<SV_B4_256, 4, SV_EPI_ANY>(w, ap, sx, M, mt0, mtn, ea, st);
    }
    if (ea.type == SV_EPI_QKV)
      return launch_mt<SV_B4_256, 2, SV_EPI_QKV>(w, ap, sx, M, mt0, mtn, ea, st);
    if (ea.type == SV_EPI_RESID)
      return launch_mt<SV_B4_256, 2, SV_EPI_RESID>(w, ap, sx, M, mt0, mtn, ea, st);
    return launch_mt<SV_B4_256, 2, SV_EPI_ANY>(w, ap, sx, M, mt0, mtn, ea, st);
  }
  if (w->type == SV_B4_32) {
    if (w->tpw == 4) return launch_mt<SV_B4_32, 4, SV_EPI_ANY>(w, ap, sx, M, mt0, mtn, ea, st);
    return launch_mt<SV_B4_32, 2, SV_EPI_ANY>(w, ap, sx, M, mt0, mtn, ea, st);
  }
  if (ea.type == SV_EPI_LM)
    return launch_mt<SV_B6_256, 2, SV_EPI_LM>(w, ap, sx, M, mt0, mtn, ea, st);
  return launch_mt<SV_B6_256, 2, SV_EPI_ANY>(w, ap, sx, M, mt0, mtn, ea, st);
}

#ifdef SV_TIMELINE
SV_TL_READER(sv_timeline_read_gemm)
#endif
