// MFMA path for experts with many routed rows (prefill chunks; page
// "GLM-5.3 Flash EXL3 for 2x DGX Sparks", "Cold prefill (E3 grouped MoE)":
// gather, gate/up + SwiGLU, down + scatter from device segment tables).
//
// One work tile = (expert, 256 routed rows, a column slice); a block is 8
// wavefronts, two per SIMD (128 accumulator registers per lane, one block per
// CU), so one wavefront's decode overlaps the other's MFMAs.  The A operand
// (activation rows) is staged through LDS in a ring of 4 stages of 32 input
// channels (prefetch distance 3).  The B operand never touches
// LDS: each lane decodes its own MFMA B fragment (8 consecutive input rows of
// one output column) straight from two code dwords into registers, so a
// wavefront decodes only the columns it owns and no decoded weight is written
// anywhere.  32-row blocks past the tile's last routed row skip their MFMAs.
//
//   gate/up : A = x (fp16) gathered through the sorted slot list; B = 2v * suh
//             (fp16, exact 2v times fp16 suh); v_mfma_f32_32x32x16_f16;
//             epilogue g = acc * svh / 128, h = silu(g) * u * suh_down -> bf16
//   down    : A = h rows (bf16, contiguous per expert); B = 2v (bf16, exact);
//             v_mfma_f32_32x32x16_bf16; epilogue y = acc * svh / 128 * w -> bf16
//             row of the slot, summed per token by the combine kernel
//   shared  : the same loop with dense fp16 nn.Linear weights as B.
//
// MFMA 32x32x16 (16-bit inputs) lane layout, lane l: A row l%32, k 8*(l/32)+0..7;
// B column l%32, k 8*(l/32)+0..7; D register r holds row 8*(r/4) + 4*(l/32) + r%4,
// column l%32.
#include "common.h"
#include "gemm.h"
#include "internal.h"
#include "trellis.h"

namespace moe {

constexpr int kBM = kTileM;    // rows per work tile
constexpr int kMB = kBM / 32;  // 32-row MFMA blocks per work tile
constexpr int kBK = 32;        // input channels per pipeline stage
constexpr int kKT = kBK / 16;  // MFMA k-steps per stage
constexpr int kRing = 4;       // LDS stages in flight (prefetch distance kRing - 1)
constexpr int kStageHalves = kBM * kBK;   // one A stage: 256 rows x 32 halves = 16 KiB
constexpr int kWaves = 8;                 // wavefronts per block (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kSlotHalves = kStageHalves + kWaves * 128;   // + one 256-byte suh area per wave


enum Mode { GATEUP_TRELLIS = 0, DOWN_TRELLIS = 1, GATEUP_DENSE = 2, DOWN_DENSE = 3 };

template <int MODE>
struct ModeTraits {
    static constexpr bool kTrellis = MODE == GATEUP_TRELLIS || MODE == DOWN_TRELLIS;
    static constexpr bool kGateUp = MODE == GATEUP_TRELLIS || MODE == GATEUP_DENSE;
    static constexpr bool kBF16 = MODE == DOWN_TRELLIS;   // MFMA input type
    // Each wavefront owns one 32-column MFMA block of one projection: for
    // gate/up, waves 0,1 hold gate and waves 2,3 up of the same 64 columns;
    // for down, 32 output columns.  A block is 4 wavefronts.
    static constexpr int kBlockN = kGateUp ? 128 : 256;
    // vector-memory instructions every wavefront issues per stage: A rows
    // (4 LDS-direct loads, plus one for suh in the trellis gate/up mode) and
    // B (trellis: 2 code dwords per k-step; dense: 16 bytes per k-step)
    static constexpr int kNA = 2 + (MODE == GATEUP_TRELLIS ? 1 : 0);
    static constexpr int kNB = kTrellis ? 2 * kKT : kKT;   // per column group
};

struct GemmArgs {
    GroupArgs g;
    // dense (shared expert) operands
    const uint16_t *dA;      // [T][Kdim] fp16 rows
    const uint16_t *dB[2];   // nn.Linear [N][Kdim] fp16
    uint16_t *dOutH;         // shared gate/up output [T][I] fp16
    float *dOutY;            // shared down output [T][H] fp32
    int64_t T;
    int nslices;             // column slices per row tile
    // trellis launches that also carry the dense shared expert: blocks from
    // routed_grid on run dense tiles with dnslices slices per row tile
    int routed_grid;
    int dnslices;
    // 4 when every routed tile has at most 64 rows (T <= 64): each block then
    // covers 4 column slices (CM = 4) and only a quarter of the slices launch
    int sdiv;
};

template <int MODE>
MOE_DEV f32x16 mfma_step(u32x4 a, u32x4 b, f32x16 c)
{
    if (ModeTraits<MODE>::kBF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}


template <int MODE, int K, int CB>
struct GemmTile {
    using TR = ModeTraits<MODE>;
    int tid, w, l, c, ts, h, pr;
    int H, I, Kdim, rows, p0, e, col;
    int64_t t0;
    // A rows: LDS-direct buffer loads; lane L of the wavefront's load j moves
    // 16 bytes of row 64w + 16j + L/4 (rows past the tile's last row repeat
    // it; their results are never stored)
    __amdgpu_buffer_rsrc_t arsrc, anull;
    uint32_t aoff[2];
    uint32_t aread[kKT];       // LDS byte offset of the lane's A fragment per k-step
    // suh (gate/up trellis): every wave fetches the 32 values of stage s of
    // its own projection with lanes 0..15 (4 bytes each) into its own
    // 256-byte area of the slot; the other lanes point past the end of the
    // buffer and read nothing.  Only the wave itself reads the area, so its
    // own vmcnt wait makes the values visible.
    __amdgpu_buffer_rsrc_t srsrc;
    uint32_t soff;
    // B: trellis codes of the lane's column, or dense weight row
    __amdgpu_buffer_rsrc_t brsrc, bnull;
    uint32_t boff0, boff1;
    uint32_t rstride;          // bytes between tile rows (trellis)
    int q;
    uint32_t m_lo, m_hi;
    // width of the wavefront's tensor and its tile bytes (K = 0: per-tensor
    // widths, read from the table; otherwise K)
    int kw;
    uint32_t tbytes;

    MOE_DEV uint32_t tile_bytes() const { return K > 0 ? (uint32_t)Tile<K>::kBytes : tbytes; }

    // raw B of one stage: CM column groups of 32 columns (trellis: 2 code
    // dwords per k-step and group; dense: 16 bytes per k-step)
    template <int CM>
    struct BRaw {
        uint32_t c[kKT][CM][2];
        u32x4 d[kKT][CM];
    };

    // Issue the A LDS-direct loads of stage s into one ring slot.  Every
    // stage issues the same loads, also past the last stage (s >= nst): those
    // go through a zero-range descriptor (no memory access; the slot they
    // fill is never read), so the count of loads in flight is the same on
    // every path through the loop and the compiler's own waits for the B
    // registers stay tight.
    MOE_DEV void load_a(int s, int nst, LDS_AS uint16_t *ring)
    {
        const __amdgpu_buffer_rsrc_t rs = s < nst ? arsrc : anull;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (LDS_AS void *)(ring + (32 * w + 16 * j) * kBK), 16, aoff[j], s * kBK * 2, 0, 0);
        if constexpr (MODE == GATEUP_TRELLIS) {
            const __amdgpu_buffer_rsrc_t ss = s < nst ? srsrc : anull;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ss, (LDS_AS void *)(ring + kStageHalves + 128 * w), 4, soff, s * kBK * 2, 0, 0);
        }
    }

    template <int CM>
    MOE_DEV void load_b(int s, int nst, BRaw<CM> &br)
    {
        const __amdgpu_buffer_rsrc_t rs = s < nst ? brsrc : bnull;
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
            if constexpr (TR::kTrellis) {
                const int so = (kKT * s + kt) * (int)rstride;
#pragma unroll
                for (int cm = 0; cm < CM; ++cm) {
                    // group cm starts two 16-column tiles further on
                    const uint32_t go = (uint32_t)cm * 2u * tile_bytes();
                    br.c[kt][cm][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, boff0 + go, so, 0);
                    br.c[kt][cm][1] = __builtin_amdgcn_raw_buffer_load_b32(rs, boff1 + go, so, 0);
                }
            } else {
                // group cm: 32 weight rows (output columns) further on
#pragma unroll
                for (int cm = 0; cm < CM; ++cm)
                    br.d[kt][cm] = __builtin_amdgcn_raw_buffer_load_b128(rs, boff0 + (uint32_t)(cm * 32 * Kdim * 2),
                                                                         (s * kBK + 16 * kt) * 2, 0);
            }
        }
    }

    // B fragment (k-step kt, column group cm) before the suh scaling: 8 exact
    // values of 2v (fp16 for gate/up, bf16 for down), or dense weights
    // K = 0 (per-tensor widths): the wavefront's width kw is a run-time,
    // wave-uniform value; only the state windows depend on it
    // (BIASED: the mcg gate/up values as 2v + 1532, see kBiasB)
    template <int KK, bool BIASED>
    MOE_DEV u32x4 decode_k(uint32_t D0, uint32_t D1) const
    {
        if constexpr (MODE == GATEUP_TRELLIS && BIASED)
            return __builtin_bit_cast(u32x4, frag_decode_f16_biased<KK>(D0, D1, q, m_lo, m_hi, kw));
        else if constexpr (MODE == GATEUP_TRELLIS)
            return __builtin_bit_cast(u32x4, frag_decode_f16<KK, CB>(D0, D1, q, m_lo, m_hi, kw));
        else
            return __builtin_bit_cast(u32x4, frag_decode_bf16<KK, CB>(D0, D1, q, m_lo, m_hi, kw));
    }

    template <int CM, bool BIASED = false>
    MOE_DEV u32x4 decode(const BRaw<CM> &br, int kt, int cm) const
    {
        if constexpr (!TR::kTrellis)
            return br.d[kt][cm];
        else
            return decode_k<K, BIASED>(br.c[kt][cm][0], br.c[kt][cm][1]);
    }

    // Gate/up tiles of one 32-row block (NMB = 1): suh multiplies the A
    // fragment, which serves all CM column groups, instead of every B
    // fragment.  With the mcg codebook B also stays biased (2v + 1532, the
    // GEMV's form, without the re-centring subtraction), and one more MFMA
    // per A fragment against a B of ones sums its row into dsum, of which the
    // epilogue takes off 1532 times.  Tiles of more blocks keep suh on B: an
    // A fragment there serves one MFMA, a B fragment NMB.
    template <int NMB>
    static constexpr bool kSuhA = MODE == GATEUP_TRELLIS && NMB == 1;
    template <int NMB>
    static constexpr bool kBiasB = kSuhA<NMB> && CB == CB_MCG;

    // Interleave the MFMAs of one fragment with the VALU work scheduled next
    // to them (the decode of the following fragment): one MFMA occupies the
    // matrix pipe for 32 cycles, in which the wave can issue ~8 VALU ops.
    template <int NMB>
    MOE_DEV static void interleave()
    {
        constexpr int kV = (NMB >= 8) ? 7 : 48 / NMB;
#pragma unroll
        for (int i = 0; i < NMB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
        }
    }

    // One pipeline stage s (ring slot SLOT = s % 4):
    //   wait for this wave's loads of stage s, barrier (every wave's loads
    //   landed, every wave is done with the slot about to be refilled),
    //   prefetch stage s + 3, read the stage's A fragments (and this wave's
    //   suh), then walk the 2 CM fragments f = (k-step, column group): the
    //   MFMAs of f (one per 32-row block) run while fragment f + 1 is decoded;
    //   the last one decodes fragment 0 of stage s + 1 (carried in dk0).
    // Loads complete in issue order and every stage issues its loads inside
    // the stage, so "at most 2 (NA + NB) outstanding" (the loads of stages
    // s + 1 and s + 2) proves that the loads of stage s are done.
    template <int NMB, int CM, int SLOT>
    MOE_DEV void stage(int s, int nst, LDS_AS uint16_t *rg, LDS_AS uint16_t *rgp, const BRaw<CM> &bcur,
                       const BRaw<CM> &bnext, BRaw<CM> &bpf, u32x4 &dk0, f32x16 acc[kMB], f32x16 &dsum)
    {
        constexpr int NA = TR::kNA, NB = TR::kNB * CM;
        constexpr bool SA = kSuhA<NMB>, BB = kBiasB<NMB>;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<2 * (NA + NB)>();
        __builtin_amdgcn_s_barrier();
        load_a(s + 3, nst, rgp);
        load_b<CM>(s + 3, nst, bpf);
        f16x8 su[kKT];
        if constexpr (MODE == GATEUP_TRELLIS) {
#pragma unroll
            for (int kt = 0; kt < kKT; ++kt)
                su[kt] = *(const LDS_AS f16x8 *)(rg + kStageHalves + 128 * (4 * pr + 2 * kt + h));
        }
        u32x4 af[kKT][NMB];
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
            for (int i = 0; i < NMB; ++i)
                af[kt][i] = *(const LDS_AS u32x4 *)((const LDS_AS char *)rg + aread[kt] + i * 32 * kBK * 2);
        if constexpr (SA) {
#pragma unroll
            for (int kt = 0; kt < kKT; ++kt)
                af[kt][0] = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, af[kt][0]) * su[kt]);
        }
        u32x4 dcur = dk0;
#pragma unroll
        for (int f = 0; f < kKT * CM; ++f) {
            const int kt = f / CM, cm = f % CM;
            u32x4 b = dcur;
            if constexpr (MODE == GATEUP_TRELLIS && !SA)
                b = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, dcur) * su[kt]);
            if (f + 1 < kKT * CM)
                dcur = decode<CM, BB>(bcur, (f + 1) / CM, (f + 1) % CM);
            else
                dcur = decode<CM, BB>(bnext, 0, 0);
            if constexpr (BB) {
                if (cm == 0) {
                    const f16x8 ones = {(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f,
                                        (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
                    dsum = mfma_step<MODE>(af[kt][0], __builtin_bit_cast(u32x4, ones), dsum);
                }
            }
#pragma unroll
            for (int i = 0; i < NMB; ++i)
                acc[cm * NMB + i] = mfma_step<MODE>(af[kt][i], b, acc[cm * NMB + i]);
            if constexpr (TR::kTrellis)
                interleave<NMB>();
        }
        dk0 = dcur;
    }

    template <int NMB, int CM>
    MOE_DEV void run(LDS_AS uint16_t *r0, LDS_AS uint16_t *r1, LDS_AS uint16_t *r2, LDS_AS uint16_t *r3,
                     f32x16 acc[kMB], f32x16 &dsum)
    {
        const int nst = Kdim / kBK;   // a multiple of 4
        BRaw<CM> b0, b1, b2, b3;
        load_a(0, nst, r0);
        load_b<CM>(0, nst, b0);
        load_a(1, nst, r1);
        load_b<CM>(1, nst, b1);
        load_a(2, nst, r2);
        load_b<CM>(2, nst, b2);
        u32x4 dk0 = decode<CM, kBiasB<NMB>>(b0, 0, 0);
        for (int s = 0; s < nst; s += 4) {
            stage<NMB, CM, 0>(s, nst, r0, r3, b0, b1, b3, dk0, acc, dsum);
            stage<NMB, CM, 1>(s + 1, nst, r1, r0, b1, b2, b0, dk0, acc, dsum);
            stage<NMB, CM, 2>(s + 2, nst, r2, r1, b2, b3, b1, dk0, acc, dsum);
            stage<NMB, CM, 3>(s + 3, nst, r3, r2, b3, b0, b2, dk0, acc, dsum);
        }
        wait_vmcnt<0>();   // the trailing zero-range loads still write LDS
    }

    // ---- the down projections' pipeline: the A fragments of a stage's first
    // k-step are read during the previous stage, so no MFMA waits for an LDS
    // read right after the barrier.  That barrier must then also cover the
    // next stage's loads, which leaves them two stages to land instead of
    // three: enough for the contiguous h rows of the down kernels, too little
    // for the gathered activation rows of gate/up (measured slower there).

    // A fragments (and, gate/up trellis, this wave's suh piece) of k-step kt
    // of the stage held in ring slot rg
    template <int NMB>
    MOE_DEV void read_a(const LDS_AS uint16_t *rg, int kt, u32x4 (&af)[NMB], f16x8 &su) const
    {
        if constexpr (MODE == GATEUP_TRELLIS)
            su = *(const LDS_AS f16x8 *)(rg + kStageHalves + 128 * (4 * pr + 2 * kt + h));
#pragma unroll
        for (int i = 0; i < NMB; ++i)
            af[i] = *(const LDS_AS u32x4 *)((const LDS_AS char *)rg + aread[kt] + i * 32 * kBK * 2);
    }

    // MFMAs of k-step kt (all CM column groups) on the fragments af, the
    // decode of the next fragment running beside each group's MFMAs
    template <int NMB, int CM>
    MOE_DEV void kstep(int kt, const u32x4 (&af)[NMB], f16x8 su, const BRaw<CM> &bcur, const BRaw<CM> &bnext,
                       u32x4 &dcur, f32x16 acc[kMB])
    {
#pragma unroll
        for (int cm = 0; cm < CM; ++cm) {
            const int f = kt * CM + cm;
            u32x4 b = dcur;
            if constexpr (MODE == GATEUP_TRELLIS)
                b = __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, dcur) * su);
            if (f + 1 < kKT * CM)
                dcur = decode<CM>(bcur, (f + 1) / CM, (f + 1) % CM);
            else
                dcur = decode<CM>(bnext, 0, 0);
#pragma unroll
            for (int i = 0; i < NMB; ++i)
                acc[cm * NMB + i] = mfma_step<MODE>(af[i], b, acc[cm * NMB + i]);
            if constexpr (TR::kTrellis)
                interleave<NMB>();
        }
    }

    // One stage s of the down pipeline (slot rg = s % 4, the next stage's slot
    // rgn, the slot rgp that stage s + 3 refills): wait for this wave's loads
    // of stage s + 1, barrier (every wave's loads of stage s + 1 landed, every
    // wave is done with rgp, last read during stage s - 1), prefetch stage
    // s + 3; k-step 0 runs on fragments read during stage s - 1 while k-step
    // 1's are read, and k-step 1 while k-step 0 of stage s + 1 is read from
    // rgn (carried in af0 / su0).  "At most NA + NB loads outstanding" (those
    // of stage s + 2) proves that the loads of stage s + 1 are done.
    template <int NMB, int CM>
    MOE_DEV void stage_ahead(int s, int nst, const LDS_AS uint16_t *rg, const LDS_AS uint16_t *rgn,
                             LDS_AS uint16_t *rgp, const BRaw<CM> &bcur, const BRaw<CM> &bnext, BRaw<CM> &bpf,
                             u32x4 &dk0, u32x4 (&af0)[NMB], f16x8 &su0, f32x16 acc[kMB])
    {
        static_assert(kKT == 2, "two k-steps per stage");
        constexpr int NA = TR::kNA, NB = TR::kNB * CM;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<NA + NB>();
        __builtin_amdgcn_s_barrier();
        load_a(s + 3, nst, rgp);
        load_b<CM>(s + 3, nst, bpf);
        u32x4 af1[NMB];
        f16x8 su1;
        read_a<NMB>(rg, 1, af1, su1);
        u32x4 dcur = dk0;
        kstep<NMB, CM>(0, af0, su0, bcur, bnext, dcur, acc);
        read_a<NMB>(rgn, 0, af0, su0);
        kstep<NMB, CM>(1, af1, su1, bcur, bnext, dcur, acc);
        dk0 = dcur;
    }

    template <int NMB, int CM>
    MOE_DEV void run_ahead(LDS_AS uint16_t *r0, LDS_AS uint16_t *r1, LDS_AS uint16_t *r2, LDS_AS uint16_t *r3,
                           f32x16 acc[kMB])
    {
        constexpr int NA = TR::kNA, NB = TR::kNB * CM;
        const int nst = Kdim / kBK;   // a multiple of 4
        BRaw<CM> b0, b1, b2, b3;
        load_a(0, nst, r0);
        load_b<CM>(0, nst, b0);
        load_a(1, nst, r1);
        load_b<CM>(1, nst, b1);
        load_a(2, nst, r2);
        load_b<CM>(2, nst, b2);
        // stage 0's data (every wave's loads) before its first fragments
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<2 * (NA + NB)>();
        __builtin_amdgcn_s_barrier();
        u32x4 af0[NMB];
        f16x8 su0;
        read_a<NMB>(r0, 0, af0, su0);
        u32x4 dk0 = decode<CM>(b0, 0, 0);
        for (int s = 0; s < nst; s += 4) {
            stage_ahead<NMB, CM>(s, nst, r0, r1, r3, b0, b1, b3, dk0, af0, su0, acc);
            stage_ahead<NMB, CM>(s + 1, nst, r1, r2, r0, b1, b2, b0, dk0, af0, su0, acc);
            stage_ahead<NMB, CM>(s + 2, nst, r2, r3, r1, b2, b3, b1, dk0, af0, su0, acc);
            stage_ahead<NMB, CM>(s + 3, nst, r3, r0, r2, b3, b0, b2, dk0, af0, su0, acc);
        }
        wait_vmcnt<0>();   // the trailing zero-range loads still write LDS
    }
};

// Column groups per wavefront for a tile of NMB 32-row blocks: small tiles
// take more columns so that every stage issues (close to) 16 MFMAs per
// wavefront, reuses each A fragment CM times and amortises its barrier and
// loads.
template <int MODE, int NMB>
struct Groups {
    static constexpr int kMax = !ModeTraits<MODE>::kTrellis ? 1 : (NMB <= 2 ? 4 : (NMB <= 4 ? 2 : 1));
};

template <int MODE, int K, int CB, int NMB, int CM>
MOE_DEV void tile_body(GemmTile<MODE, K, CB> &g, const GemmArgs &args, int n0,
                       uint16_t *ring0, uint16_t *ring1, uint16_t *ring2, uint16_t *ring3)
{
    using TR = ModeTraits<MODE>;
    const GroupArgs &a = args.g;
    // ---- B source: lane -> (column c of tile ts, k-half h); the wavefront
    // owns CM groups of 32 columns of one projection over all 256 rows:
    // gate/up -> waves 0,1 gate and waves 2,3 up of the block's 64 CM
    // intermediate columns; down -> 32 CM of the block's 128 CM output columns
    const int Nout = TR::kGateUp ? g.I : g.H;
    g.col = (TR::kGateUp ? n0 + 32 * CM * (g.w & 3) : n0 + 32 * CM * g.w) + 16 * g.ts + g.c;
    if constexpr (TR::kTrellis) {
        const TensorCodes tcs = tensor_codes<K>(a, g.pr, g.e, g.Kdim, Nout);
        g.kw = K > 0 ? K : __builtin_amdgcn_readfirstlane(tcs.K);
        g.tbytes = 32u * (uint32_t)g.kw;
        int d0, d1, q;
        frag_pos_rt(g.kw, g.c, g.h, d0, d1, q);
        g.q = q;
        g.rstride = (uint32_t)(Nout / 16) * g.tile_bytes();
        g.brsrc = buf_rsrc(tcs.base, tcs.bytes);
        g.bnull = buf_rsrc(tcs.base, 0);
        const uint32_t tile0 = (uint32_t)(g.col / 16) * g.tile_bytes();
        g.boff0 = tile0 + 4 * d0;
        g.boff1 = tile0 + 4 * d1;
        g.srsrc = g.bnull;
        g.soff = 0;
        if constexpr (MODE == GATEUP_TRELLIS) {
            // piece w & 3 (k = 8 (w & 3) .. + 7 of the stage) of projection w >> 2
            g.srsrc = buf_rsrc(a.suh[g.pr] + (int64_t)g.e * g.H + 8 * (g.w & 3),
                               (uint32_t)(g.H * 2 - 16 * (g.w & 3)));
            g.soff = g.l < 4 ? 4u * g.l : 0x7FFFFFF0u;
        }
    } else {
        const uint16_t *W = TR::kGateUp ? args.dB[g.pr] : args.dB[0];
        g.brsrc = buf_rsrc(W, (uint32_t)((int64_t)Nout * g.Kdim * 2));
        g.bnull = buf_rsrc(W, 0);
        g.srsrc = g.bnull;
        g.soff = 0;
        g.boff0 = (uint32_t)(((int64_t)g.col * g.Kdim + 8 * g.h) * 2);
        g.boff1 = 0;
        g.rstride = 0;
    }

    LDS_AS uint16_t *R0 = (LDS_AS uint16_t *)ring0, *R1 = (LDS_AS uint16_t *)ring1;
    LDS_AS uint16_t *R2 = (LDS_AS uint16_t *)ring2, *R3 = (LDS_AS uint16_t *)ring3;
    f32x16 acc[kMB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
        acc[i] = (f32x16){};
    f32x16 dsum = {};
    if constexpr (TR::kGateUp)
        g.template run<NMB, CM>(R0, R1, R2, R3, acc, dsum);
    else
        g.template run_ahead<NMB, CM>(R0, R1, R2, R3, acc);
    __syncthreads();   // every wave is done with the rings (reused below)

    // the biased gate/up accumulators of one-block tiles: 1532 x row sum off
    auto accv = [&](int b, int r) -> float {
        if constexpr (GemmTile<MODE, K, CB>::template kBiasB<NMB>)
            return acc[b][r] - 1532.0f * dsum[r];
        else
            return acc[b][r];
    };
    // ---- epilogue.  Accumulator block b = cm * NMB + i covers rows 32 i + ..
    // of column group cm; its D register r holds row 32i + 8(r/4) + 4h + r%4.
    constexpr int NB = NMB * CM;
    const int h = g.h, rows = g.rows, e = g.e, p0 = g.p0;
    const int H = g.H, I = g.I;
    const int64_t t0 = g.t0;
    const int mblocks = (rows + 31) >> 5;
    if constexpr (TR::kGateUp) {
        // gate wavefront w and up wavefront w + 4 hold the same columns.  In
        // rounds of four accumulator blocks, the up wavefront hands its scaled
        // values of the first two blocks to the gate wavefront through LDS and
        // the gate wavefront its scaled values of the last two to the up
        // wavefront; each then finishes its two blocks (block b of column group
        // cg = w & 3 goes to ring cg at 4 KiB per block).
        const int cg = g.w & 3;
        float *ex = cg == 0 ? (float *)ring0 : cg == 1 ? (float *)ring1 : cg == 2 ? (float *)ring2 : (float *)ring3;
#pragma unroll
        for (int round = 0; round < (NB + 3) / 4; ++round) {
#pragma unroll
            for (int b = 4 * round; b < 4 * round + 4 && b < NB; ++b) {
                const int cm = b / NMB, i = b % NMB;
                const int col = g.col + 32 * cm;
                // blocks 0, 1 of the round are finished by the gate wavefront
                const bool mine = (g.pr == 0) == ((b & 3) < 2);
                if (!mine && i < mblocks) {
                    const float sc = MODE != GATEUP_TRELLIS ? 1.0f
                                     : f16_to_f32(a.svh[g.pr][(int64_t)e * I + col]) * (1.0f / 128.0f);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        ex[((b & 3) * 16 + r) * 64 + g.l] = accv(b, r) * sc;
                }
            }
            __syncthreads();
#pragma unroll
            for (int b = 4 * round; b < 4 * round + 4 && b < NB; ++b) {
                const int cm = b / NMB, i = b % NMB;
                const int col = g.col + 32 * cm;
                const bool mine = (g.pr == 0) == ((b & 3) < 2);
                if (mine && i < mblocks) {
                    float sg = 1.0f, su = 1.0f, sd = 1.0f;
                    if constexpr (MODE == GATEUP_TRELLIS) {
                        sg = f16_to_f32(a.svh[0][(int64_t)e * I + col]) * (1.0f / 128.0f);
                        su = f16_to_f32(a.svh[1][(int64_t)e * I + col]) * (1.0f / 128.0f);
                        sd = f16_to_f32(a.suh[2][(int64_t)e * I + col]);
                    }
                    float hv[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float other = ex[((b & 3) * 16 + r) * 64 + g.l];
                        const float gv = g.pr == 0 ? accv(b, r) * sg : other;
                        const float uv = g.pr == 0 ? other : accv(b, r) * su;
                        hv[r] = silu_f(gv) * uv * sd;
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (row < rows) {
                            if constexpr (MODE == GATEUP_TRELLIS)
                                a.hbuf[(int64_t)(p0 + row) * I + col] = f32_to_bf16_bits(hv[r]);
                            else
                                args.dOutH[(t0 + row) * I + col] = f32_to_f16_bits(hv[r]);
                        }
                    }
                }
            }
            __syncthreads();
        }
    } else {
        // down: the tile's slot ids and routing weights come through LDS (one
        // row per thread, the rings being free now) rather than as two
        // dependent global loads for every accumulator element
        LDS_AS int *slots = (LDS_AS int *)R0;
        LDS_AS float *wts = (LDS_AS float *)(R0 + 2 * kBM);
        if constexpr (MODE == DOWN_TRELLIS) {
            if (g.tid < rows) {
                const int slot = a.sorted[p0 + g.tid];
                slots[g.tid] = slot;
                wts[g.tid] = a.w[slot];
            }
            __syncthreads();
        }
        // each wavefront turns a 32 x 32 accumulator block into bf16 rows in
        // its own 2 KiB of ring 1, then stores 16 bytes per lane of a row
        LDS_AS uint16_t *tw = R1 + 1024 * g.w;
        const int lc = g.l & 31;
#pragma unroll
        for (int cm = 0; cm < CM; ++cm) {
            const int col = g.col + 32 * cm;
            const float sv = MODE == DOWN_TRELLIS ? f16_to_f32(a.svh[2][(int64_t)e * H + col]) * (1.0f / 128.0f) : 1.0f;
#pragma unroll
            for (int i = 0; i < NMB; ++i) {
                const int b = cm * NMB + i;
                if (i < mblocks) {
                    if constexpr (MODE == DOWN_TRELLIS) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int rl = 8 * (r >> 2) + 4 * h + (r & 3);
                            tw[rl * 32 + lc] = f32_to_bf16_bits(acc[b][r] * sv * wts[32 * i + rl]);
                        }
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const int rl = (g.l >> 2) + 16 * q, row = 32 * i + rl;
                            const u32x4 v = *(const LDS_AS u32x4 *)(tw + rl * 32 + 8 * (g.l & 3));
                            if (row < rows)
                                *(u32x4 *)(a.ybuf + (int64_t)slots[row] * H + (col - lc) + 8 * (g.l & 3)) = v;
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                            if (row < rows)
                                args.dOutY[(t0 + row) * H + col] = acc[b][r];
                        }
                    }
                }
            }
        }
    }
    static_assert(NB <= kMB, "accumulator blocks");
}

// One block's work: block L of a grid with `nslices` column slices per row
// tile, of which nslices / sdiv are launched (sdiv > 1 only where every tile
// takes sdiv column groups per wavefront).
template <int MODE, int K, int CB>
MOE_DEV void block_body(const GemmArgs &args, int L, int nslices, int sdiv, uint16_t *ring0, uint16_t *ring1,
                        uint16_t *ring2, uint16_t *ring3)
{
    using TR = ModeTraits<MODE>;
    const GroupArgs &a = args.g;
    GemmTile<MODE, K, CB> g;
    g.tid = threadIdx.x;
    g.w = __builtin_amdgcn_readfirstlane(g.tid >> 6);   // wave-uniform
    g.l = g.tid & 63;
    g.H = a.H;
    g.I = a.I;
    g.Kdim = TR::kGateUp ? g.H : g.I;

    // ---- work tile; `nslices` counts column slices at one group per wave
    int ti, slice;
    xcd_map(L, nslices / sdiv, ti, slice);
    g.e = 0;
    g.p0 = 0;
    g.t0 = 0;
    if constexpr (TR::kTrellis) {
        if (ti >= a.hdr->n_tiles)
            return;
        g.e = a.tiles[2 * ti];
        const int m0 = a.tiles[2 * ti + 1];
        g.rows = min(kBM, a.counts[g.e] - m0);
        g.p0 = a.offsets[g.e] + m0;
    } else {
        g.t0 = (int64_t)ti * kBM;
        if (g.t0 >= args.T)
            return;
        g.rows = (int)min<int64_t>(kBM, args.T - g.t0);
    }
    const int mblocks = (g.rows + 31) >> 5;
    // column groups per wavefront for this tile (a slice beyond the tile's
    // share has no work: the whole block leaves before any barrier)
    int cm = 1;
    if (TR::kTrellis && mblocks <= 2)
        cm = (nslices % 4 == 0) ? 4 : (nslices % 2 == 0) ? 2 : 1;
    else if (TR::kTrellis && mblocks <= 4)
        cm = (nslices % 2 == 0) ? 2 : 1;
    if (slice >= nslices / cm)
        return;
    const int n0 = slice * TR::kBlockN * cm;

    // ---- A rows
    {
        const uint16_t *abase;
        uint32_t abytes;
        if constexpr (MODE == GATEUP_TRELLIS) {
            abase = a.x16;
            abytes = (uint32_t)(a.T * (int64_t)g.H * 2);
        } else if constexpr (MODE == DOWN_TRELLIS) {
            abase = a.hbuf + (int64_t)g.p0 * g.I;
            abytes = (uint32_t)((int64_t)g.rows * g.I * 2);
        } else {
            abase = args.dA + g.t0 * g.Kdim;
            abytes = (uint32_t)((int64_t)g.rows * g.Kdim * 2);
        }
        g.arsrc = buf_rsrc(abase, abytes);
        g.anull = buf_rsrc(abase, 0);
        // rows past the tile's last 32-row block feed no stored result: the
        // waves that would load them go through the zero-range descriptor
        if (g.w >= mblocks)
            g.arsrc = g.anull;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 32 * g.w + 16 * j + (g.l >> 2);
            const int rc = min(r, g.rows - 1);
            int64_t row;
            if constexpr (MODE == GATEUP_TRELLIS)
                row = slot_token(a.sorted[g.p0 + rc], a.nr, a.k);
            else
                row = rc;
            const int piece = a_slot(r, g.l & 3);   // slot l&3 holds this k piece
            g.aoff[j] = (uint32_t)((row * g.Kdim + 8 * piece) * 2);
        }
        g.h = g.l >> 5;
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
            const int r = g.l & 31;
            g.aread[kt] = (uint32_t)(r * kBK * 2 + 16 * a_slot(r, 2 * kt + g.h));
        }
    }
    g.c = g.l & 15;
    g.ts = (g.l >> 4) & 1;
    g.pr = TR::kGateUp ? g.w >> 2 : 2;
    g.m_lo = a.mcg & 0xFFFFu;
    g.m_hi = a.mcg >> 16;
    g.q = 0;

    if (mblocks <= 1) {
        if (cm == 4)
            tile_body<MODE, K, CB, 1, Groups<MODE, 1>::kMax>(g, args, n0, ring0, ring1, ring2, ring3);
        else if (cm == 2)
            tile_body<MODE, K, CB, 1, (Groups<MODE, 1>::kMax > 2 ? 2 : Groups<MODE, 1>::kMax)>(g, args, n0, ring0, ring1, ring2, ring3);
        else
            tile_body<MODE, K, CB, 1, 1>(g, args, n0, ring0, ring1, ring2, ring3);
    } else if (mblocks <= 2) {
        if (cm == 4)
            tile_body<MODE, K, CB, 2, Groups<MODE, 2>::kMax>(g, args, n0, ring0, ring1, ring2, ring3);
        else if (cm == 2)
            tile_body<MODE, K, CB, 2, (Groups<MODE, 2>::kMax > 2 ? 2 : Groups<MODE, 2>::kMax)>(g, args, n0, ring0, ring1, ring2, ring3);
        else
            tile_body<MODE, K, CB, 2, 1>(g, args, n0, ring0, ring1, ring2, ring3);
    } else if (mblocks <= 4) {
        if (cm == 2)
            tile_body<MODE, K, CB, 4, Groups<MODE, 4>::kMax>(g, args, n0, ring0, ring1, ring2, ring3);
        else
            tile_body<MODE, K, CB, 4, 1>(g, args, n0, ring0, ring1, ring2, ring3);
    } else if (mblocks <= 6) {
        tile_body<MODE, K, CB, 6, 1>(g, args, n0, ring0, ring1, ring2, ring3);
    } else {
        tile_body<MODE, K, CB, 8, 1>(g, args, n0, ring0, ring1, ring2, ring3);
    }
}

template <int MODE, int K, int CB>
__global__ __launch_bounds__(kThreads, 1) void group_gemm_kernel(GemmArgs args)
{
    // four ring slots, each one A stage plus four 256-byte suh areas (used in
    // the trellis gate/up mode); four distinct LDS objects let the compiler
    // tell the slots' LDS-direct writes apart
    __shared__ __align__(16) uint16_t ring0[kSlotHalves];
    __shared__ __align__(16) uint16_t ring1[kSlotHalves];
    __shared__ __align__(16) uint16_t ring2[kSlotHalves];
    __shared__ __align__(16) uint16_t ring3[kSlotHalves];
    if constexpr (ModeTraits<MODE>::kTrellis) {
        // blocks past the routed experts' grid run tiles of the dense shared
        // expert, so its work fills the CUs the routed tiles leave idle at the
        // end of the launch (routed_grid is a multiple of 8: XCD order holds)
        if ((int)blockIdx.x >= args.routed_grid) {
            constexpr int DM = MODE == GATEUP_TRELLIS ? GATEUP_DENSE : DOWN_DENSE;
            block_body<DM, K, CB>(args, (int)blockIdx.x - args.routed_grid, args.dnslices, 1, ring0, ring1, ring2,
                                  ring3);
            return;
        }
    }
    block_body<MODE, K, CB>(args, (int)blockIdx.x, args.nslices, args.sdiv > 1 ? args.sdiv : 1, ring0, ring1, ring2,
                            ring3);
}

template <int MODE>
static hipError_t launch_grid(const GemmArgs &ga, unsigned grid, hipStream_t s)
{
    const GroupArgs &a = ga.g;
    if (grid == 0)
        return hipSuccess;
    if constexpr (ModeTraits<MODE>::kTrellis) {
        if (a.code_tab && a.cb == 0) group_gemm_kernel<MODE, 0, 0><<<grid, kThreads, 0, s>>>(ga);
        else if (a.code_tab) group_gemm_kernel<MODE, 0, 1><<<grid, kThreads, 0, s>>>(ga);
        else if (a.K == 2 && a.cb == 0) group_gemm_kernel<MODE, 2, 0><<<grid, kThreads, 0, s>>>(ga);
        else if (a.K == 3 && a.cb == 0) group_gemm_kernel<MODE, 3, 0><<<grid, kThreads, 0, s>>>(ga);
        else if (a.K == 4 && a.cb == 0) group_gemm_kernel<MODE, 4, 0><<<grid, kThreads, 0, s>>>(ga);
        else if (a.K == 2) group_gemm_kernel<MODE, 2, 1><<<grid, kThreads, 0, s>>>(ga);
        else if (a.K == 3) group_gemm_kernel<MODE, 3, 1><<<grid, kThreads, 0, s>>>(ga);
        else group_gemm_kernel<MODE, 4, 1><<<grid, kThreads, 0, s>>>(ga);
    } else {
        group_gemm_kernel<MODE, 2, 0><<<grid, kThreads, 0, s>>>(ga);
    }
    return hipGetLastError();
}

// Blocks for `tiles` row tiles at `nslices` slices each, in whole XCD rounds.
static unsigned grid_of(int tiles, int nslices)
{
    return tiles > 0 ? (unsigned)(((tiles + 7) / 8) * 8 * nslices) : 0u;
}

static int dense_tiles(int64_t T) { return (int)((T + kBM - 1) / kBM); }

hipError_t launch_mfma_gateup(const GroupArgs &a, int max_tiles, const SharedArgs *sh, hipStream_t s)
{
    GemmArgs ga{};
    ga.g = a;
    ga.nslices = a.I / ModeTraits<GATEUP_TRELLIS>::kBlockN;
    ga.sdiv = (a.T <= 64 && ga.nslices % 4 == 0) ? 4 : 1;
    ga.routed_grid = (int)grid_of(max_tiles, ga.nslices / ga.sdiv);
    unsigned grid = (unsigned)ga.routed_grid;
    if (sh) {
        ga.dA = sh->x16;
        ga.dB[0] = sh->w[0];
        ga.dB[1] = sh->w[1];
        ga.dOutH = sh->h;
        ga.T = a.T;
        ga.dnslices = a.I / ModeTraits<GATEUP_DENSE>::kBlockN;
        grid += grid_of(dense_tiles(a.T), ga.dnslices);
    }
    return launch_grid<GATEUP_TRELLIS>(ga, grid, s);
}

hipError_t launch_mfma_down(const GroupArgs &a, int max_tiles, const SharedArgs *sh, hipStream_t s)
{
    GemmArgs ga{};
    ga.g = a;
    ga.nslices = a.H / ModeTraits<DOWN_TRELLIS>::kBlockN;
    ga.sdiv = (a.T <= 64 && ga.nslices % 4 == 0) ? 4 : 1;
    ga.routed_grid = (int)grid_of(max_tiles, ga.nslices / ga.sdiv);
    unsigned grid = (unsigned)ga.routed_grid;
    if (sh) {
        ga.dA = sh->h;
        ga.dB[0] = sh->w[2];
        ga.dOutY = sh->y;
        ga.T = a.T;
        ga.dnslices = a.H / ModeTraits<DOWN_DENSE>::kBlockN;
        grid += grid_of(dense_tiles(a.T), ga.dnslices);
    }
    return launch_grid<DOWN_TRELLIS>(ga, grid, s);
}

hipError_t launch_shared_gateup(const uint16_t *x16, int64_t T, int H, int I, const uint16_t *wg,
                                const uint16_t *wu, uint16_t *sh, hipStream_t s)
{
    GemmArgs ga{};
    ga.g.H = H;
    ga.g.I = I;
    ga.dA = x16;
    ga.dB[0] = wg;
    ga.dB[1] = wu;
    ga.dOutH = sh;
    ga.T = T;
    ga.nslices = I / ModeTraits<GATEUP_DENSE>::kBlockN;
    ga.sdiv = 1;
    return launch_grid<GATEUP_DENSE>(ga, grid_of(dense_tiles(T), ga.nslices), s);
}

hipError_t launch_shared_down(const uint16_t *sh, int64_t T, int H, int I, const uint16_t *wd,
                              float *sy, hipStream_t s)
{
    GemmArgs ga{};
    ga.g.H = H;
    ga.g.I = I;
    ga.dA = sh;
    ga.dB[0] = wd;
    ga.dOutY = sy;
    ga.T = T;
    ga.nslices = H / ModeTraits<DOWN_DENSE>::kBlockN;
    ga.sdiv = 1;
    return launch_grid<DOWN_DENSE>(ga, grid_of(dense_tiles(T), ga.nslices), s);
}

}  // namespace moe
