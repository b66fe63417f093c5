// lora_shrink.hip -- buf[i][t][:] += scale * x[t] @ A_i[id_t]^T for tokens
// grouped by LoRA id (PunicaWrapperGPU.add_shrink on the "punica_gpu" page).
//
// Each segment (the tokens of one id, contiguous in the sorted index list) is
// a skinny GEMM  C[rows = S*r][tokens] = A_id[rows][H] * X_seg[tokens][H]^T
// run on the bf16 MFMA (v_mfma_f32_16x16x32_bf16) with the weight rows on the
// M side and the gathered token rows on the N side, so that every lane ends up
// with 4 consecutive rank entries of one token: 16-byte stores into buf.
//
// Work unit = (token tile of a segment, block of weight rows, K chunk), in a
// canonical tile-major order that is cut into one contiguous chunk per XCD
// (neighbouring units share x rows or weight rows through that XCD's L2).
// The grid is persistent: each workgroup builds the tile table in LDS once and
// walks its chunk.  A workgroup has 4 waves laid out as WR (row groups) x WK
// (K interleave); each wave streams its weight rows and the tile's token rows
// from HBM straight into MFMA operand registers: every lane loads 32
// contiguous bytes of a row per 64-wide K step (4 lanes cover one 128-byte
// line), feeding two MFMAs (the same K permutation on both operands leaves
// the sum unchanged).
//
// All loads are unconditional: lanes of missing tokens or rows read a clamped
// valid row (their outputs are discarded), and only the last K step of a
// ragged K range is masked.  With a fixed number of loads per step the
// compiler can wait for exactly the step being multiplied while the next one
// is in flight.  Partial sums of the WK waves are added in LDS; K chunks are
// combined with float atomics, else the unit does a read-modify-write of buf
// (or, for a fresh buffer, a plain store).
#include "lora_internal.h"

#include <stdlib.h>

namespace lora {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Loads of one 64-wide K step: 16 elements of each row at kk (clamped to the
// row start where the step runs past kend; those halves are masked later).
template <int N>
__device__ __forceinline__ void load_step(const uint16_t *const (&row)[N], int kk, int kend, u32x4 (&v)[N][2]) {
    const int o0 = kk + 8 <= kend ? kk : 0;
    const int o1 = kk + 16 <= kend ? kk + 8 : 0;
#pragma unroll
    for (int q = 0; q < N; ++q) {
        v[q][0] = ld16(row[q] + o0);
        v[q][1] = ld16(row[q] + o1);
    }
}

template <int N>
__device__ __forceinline__ void mask_step(int kk, int kend, u32x4 (&v)[N][2]) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool ok0 = kk + 8 <= kend, ok1 = kk + 16 <= kend;
#pragma unroll
    for (int q = 0; q < N; ++q) {
        v[q][0] = ok0 ? v[q][0] : z;
        v[q][1] = ok1 ? v[q][1] : z;
    }
}

template <int NT, int MT, int WK>
__global__ __launch_bounds__(kThreads) void shrink_kernel(ShrinkArgs a) {
    prefetch_kernargs<ShrinkArgs>();
    constexpr int WR = 4 / WK;
    constexpr int kTileTokens = 16 * NT;
    extern __shared__ int smem[];
    __shared__ int s_wsum[kThreads / kWave];
    __shared__ floatx4 red[(WK > 1 ? WK - 1 : 1) * WR * MT * NT * kWave];

    const int nslots = a.meta.nslots;
    const int total = build_tile_table<kThreads>(a.meta, kTileTokens, smem, s_wsum);

    const int lane = lane_id(), wave = wave_id();
    const int wk = wave % WK, wr = wave / WK;
    const int col = lane & 15, g = lane >> 4;
    const int rows_per_wg = WR * MT * 16;
    const bool atomic = a.k_splits > 1;

    const UnitWalker walk(total * a.row_blocks * a.k_splits);
    for (int jj = walk.first;; jj += walk.stride) {
        const int u = walk.unit(jj);
        if (u < 0) break;
        const int ks = u % a.k_splits;
        const int rest = u / a.k_splits;
        const int rb = rest % a.row_blocks;
        const TileRef tr = lookup_tile(smem, nslots, rest / a.row_blocks);

        // token rows (N side); missing tokens repeat the segment's last token
        const uint16_t *xrow[NT];
        int tok[NT];
        bool tv[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int p = tr.tile * kTileTokens + nt * 16 + col;
            tv[nt] = p < tr.seg_count;
            int t = sorted_at(a.meta, smem, tr.seg_start + (tv[nt] ? p : tr.seg_count - 1));
            if ((unsigned)t >= (unsigned)a.num_tokens) {   // metadata not from this batch
                t = 0;
                tv[nt] = false;
            }
            tok[nt] = t;
            xrow[nt] = a.x + (int64_t)t * a.ldx;
        }
        // weight rows (M side); rows past S*r repeat the last row
        const uint16_t *arow[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            int row = rb * rows_per_wg + (wr * MT + mt) * 16 + col;
            row = row < a.rows ? row : a.rows - 1;
            const int i = row / a.rank, j = row - i * a.rank;
            arow[mt] = select_slice(a.a, i) + ((int64_t)tr.lora_id * a.rank + j) * a.hidden;
        }

        const int kbeg = ks * a.k_chunk;
        const int kend = min(kbeg + a.k_chunk, a.hidden);
        const int nsteps = (kend - kbeg + 63) / 64;
        const bool ragged = ((kend - kbeg) & 63) != 0;

        floatx4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

        u32x4 av[MT][2], xv[NT][2];
        {
            const int kk = kbeg + min(wk, nsteps - 1) * 64 + g * 16;
            load_step<MT>(arow, kk, kend, av);
            load_step<NT>(xrow, kk, kend, xv);
        }
        for (int s = wk; s < nsteps; s += WK) {
            // prefetch the next step (the last step is re-read, never skipped)
            u32x4 an[MT][2], xn[NT][2];
            const int kn = kbeg + min(s + WK, nsteps - 1) * 64 + g * 16;
            load_step<MT>(arow, kn, kend, an);
            load_step<NT>(xrow, kn, kend, xn);
            if (ragged && s == nsteps - 1) {
                const int kk = kbeg + s * 64 + g * 16;
                mask_step<MT>(kk, kend, av);
                mask_step<NT>(kk, kend, xv);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[mt][nt] = mfma16x16x32(as_bf16x8(av[mt][h]), as_bf16x8(xv[nt][h]), acc[mt][nt]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                av[mt][0] = an[mt][0];
                av[mt][1] = an[mt][1];
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                xv[nt][0] = xn[nt][0];
                xv[nt][1] = xn[nt][1];
            }
        }

        bool writer = true;
        if constexpr (WK > 1) {
            if (wk > 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        red[(((wk - 1) * WR + wr) * MT * NT + mt * NT + nt) * kWave + lane] = acc[mt][nt];
            }
            __syncthreads();
            if (wk == 0) {
#pragma unroll
                for (int w = 1; w < WK; ++w)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            acc[mt][nt] += red[(((w - 1) * WR + wr) * MT * NT + mt * NT + nt) * kWave + lane];
            }
            __syncthreads();   // `red` is rewritten by the next unit
            writer = wk == 0;
        }

        // D layout: lane holds rows 4g..4g+3 of the m-tile for token column `col`.
        // With accumulation every old value is loaded before the first store
        // (a store between them would make each load wait for the previous one).
        if (writer) {
            float *row_ptr[MT];
            bool rv[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row0 = rb * rows_per_wg + (wr * MT + mt) * 16 + 4 * g;
                rv[mt] = row0 < a.rows;
                const int r = rv[mt] ? row0 : 0;
                const int i = r / a.rank, j = r - i * a.rank;
                row_ptr[mt] = a.buf + (int64_t)i * a.num_tokens * a.rank + j;
            }
            auto dst = [&](int mt, int nt) { return row_ptr[mt] + (int64_t)tok[nt] * a.rank; };
            if (!atomic && !a.overwrite) {
                constexpr int G = NT < 2 ? NT : 2;   // n-tiles per round trip
#pragma unroll
                for (int n0 = 0; n0 < NT; n0 += G) {
                    floatx4 old[MT][G];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int q = 0; q < G; ++q)
                            if (rv[mt] && tv[n0 + q]) old[mt][q] = *reinterpret_cast<const floatx4 *>(dst(mt, n0 + q));
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int q = 0; q < G; ++q)
                            if (rv[mt] && tv[n0 + q])
                                *reinterpret_cast<floatx4 *>(dst(mt, n0 + q)) = old[mt][q] + acc[mt][n0 + q] * a.scale;
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        if (!rv[mt] || !tv[nt]) continue;
                        float *d = dst(mt, nt);
                        const floatx4 v = acc[mt][nt] * a.scale;
                        if (atomic) {
                            unsafeAtomicAdd(d + 0, v[0]);
                            unsafeAtomicAdd(d + 1, v[1]);
                            unsafeAtomicAdd(d + 2, v[2]);
                            unsafeAtomicAdd(d + 3, v[3]);
                        } else {
                            *reinterpret_cast<floatx4 *>(d) = v;
                        }
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// LDS-staged variant for tiles of many tokens (prefill-like segments).
//
// A workgroup computes a tile of BT = 16*NT tokens x BR = 16*MR weight rows
// over its K range.  Every 64-wide K step, the tile's BT token rows and BR
// weight rows (128 bytes each) are copied from HBM straight into LDS with
// global_load_lds_dwordx4: 8 lanes cover one row's 128 bytes, so each wave
// instruction moves 8 whole row segments (1 KB, fully coalesced), and every
// element is fetched once per workgroup.  The 16-byte chunks of row r are
// stored XOR-swizzled (chunk c at slot c ^ (r & 7)) so that the MFMA operand
// reads (ds_read_b128 of one chunk from 8 different rows) hit 8 different
// bank groups.  All STAGES stages are filled ahead; a wave waits only for the
// step it is about to use (s_waitcnt vmcnt), then a barrier publishes the step
// to the whole workgroup.  Once every wave has read its MFMA operands of the
// step into registers, a second barrier frees the stage and the step STAGES
// ahead is issued into it before the MFMAs run, so that STAGES steps stay in
// flight behind the arithmetic.  Waves split the tile as WR row groups x
// (4 / WR) token groups; each output element belongs to one wave, so K
// chunks are combined only across workgroups, never inside one.
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// 16-byte LDS read issued as an opaque instruction: the stage protocol
// (s_waitcnt vmcnt + barrier) already orders it after the direct-to-LDS
// loads that filled the stage, and the compiler would otherwise wait for
// every load in flight before each read.  Callers wait with lds_wait().
__device__ __forceinline__ u32x4 lds_read16(const unsigned char *p) {
    u32x4 r;
    const uint32_t addr = (uint32_t)(uintptr_t)p;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
    return r;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Ties a register to the preceding lds_wait(): its consumers cannot be
// scheduled above the wait (the value is an output of this statement).
__device__ __forceinline__ void after_wait(u32x4 &v) { asm volatile("" : "+v"(v)); }

// The tile of one piece of work and where its sums go: BT = 16*NT tokens x
// BR = 16*MR weight rows, the waves split as WR row groups x (4 / WR) token
// groups, each wave holding MT x NTW accumulator tiles of 16 x 16.
template <int NT, int MR, int WR>
struct TileLayout {
    static constexpr int WC = 4 / WR;
    static constexpr int BT = 16 * NT, BR = 16 * MR;
    static constexpr int MT = MR / WR, NTW = NT / WC;
    static constexpr int SLOT = BT * BR;        // floats of one tile's partial sums
    static_assert(MR % WR == 0 && NT % WC == 0, "tile shape");
    struct Acc {
        floatx4 v[MT][NTW];
    };

    // Writes the piece's sums into buf, scaled.  Every load comes before the
    // stores it could precede: the tile's token indices first, and with
    // accumulation the old values of a group of n-tiles before that group's
    // stores (a store between loads would make each load wait for the one
    // before it, a memory round trip per 16 x 16 tile).
    __device__ __forceinline__ static void store(const ShrinkArgs &a, const TileRef &tr, int rb,
                                                 const floatx4 (&acc)[MT][NTW], bool atomic) {
        const int lane = lane_id(), wave = wave_id();
        const int wr = wave % WR, wc = wave / WR;
        const int n16 = lane & 15, g = lane >> 4;
        // D layout: lane holds rows 4g..4g+3 of m-tile mt for token column n16 of n-tile nt
        int tok[NTW];
        bool tv[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int p = tr.tile * BT + (wc * NTW + nt) * 16 + n16;
            tok[nt] = a.meta.sorted[tr.seg_start + (p < tr.seg_count ? p : tr.seg_count - 1)];
            tv[nt] = p < tr.seg_count;
        }
        float *row_ptr[MT];
        bool rv[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row0 = rb * BR + (wr * MT + mt) * 16 + 4 * g;
            rv[mt] = row0 < a.rows;
            const int r = rv[mt] ? row0 : 0;
            const int i = r / a.rank, jr = r - i * a.rank;
            row_ptr[mt] = a.buf + (int64_t)i * a.num_tokens * a.rank + jr;
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) tv[nt] = tv[nt] && (unsigned)tok[nt] < (unsigned)a.num_tokens;
        auto dst = [&](int mt, int nt) { return row_ptr[mt] + (int64_t)tok[nt] * a.rank; };
        if (atomic || a.overwrite) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                if (!tv[nt]) continue;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (!rv[mt]) continue;
                    float *d = dst(mt, nt);
                    const floatx4 v = acc[mt][nt] * a.scale;
                    if (atomic) {
                        unsafeAtomicAdd(d + 0, v[0]);
                        unsafeAtomicAdd(d + 1, v[1]);
                        unsafeAtomicAdd(d + 2, v[2]);
                        unsafeAtomicAdd(d + 3, v[3]);
                    } else {
                        *reinterpret_cast<floatx4 *>(d) = v;
                    }
                }
            }
            return;
        }
        // n-tiles per round trip: all of them when their old values fit in 24
        // 16-byte registers, else 4
        constexpr int G = MT * NTW <= 24 ? NTW : (NTW < 4 ? NTW : 4);
#pragma unroll
        for (int n0 = 0; n0 < NTW; n0 += G) {
            floatx4 old[G][MT];
#pragma unroll
            for (int q = 0; q < G; ++q)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    if (n0 + q < NTW && tv[n0 + q] && rv[mt])
                        old[q][mt] = *reinterpret_cast<const floatx4 *>(dst(mt, n0 + q));
#pragma unroll
            for (int q = 0; q < G; ++q)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    if (n0 + q < NTW && tv[n0 + q] && rv[mt])
                        *reinterpret_cast<floatx4 *>(dst(mt, n0 + q)) = old[q][mt] + acc[mt][n0 + q] * a.scale;
        }
    }
};

// The LDS-staged pipeline of one piece of work, shared by the unit-walking
// and the stream-K kernels: the tile `tr`, the weight rows of row block `rb`,
// the K range [kbeg, kend).
template <int NT, int MR, int WR, int STAGES>
struct Staged : TileLayout<NT, MR, WR> {
    using L = TileLayout<NT, MR, WR>;
    using typename L::Acc;
    using L::BT;
    using L::BR;
    using L::MT;
    using L::NTW;
    static constexpr int NSTAGE = STAGES;
    static constexpr int ROWS = BT + BR;
    static constexpr int INSTR = ROWS / 32;     // load instructions per wave per step
    static_assert(ROWS % 32 == 0, "tile shape");
    static_assert(STAGES * INSTR < 64, "vmcnt range");
    typedef unsigned char Stage[ROWS * 128];

    // A piece's source rows and K range.  The runner has three phases:
    //   sources  loads the sorted indices of the piece's token rows;
    //   prime    turns them into row pointers and issues the first STAGES
    //            steps;
    //   finish   runs every step and drains the pipeline.
    struct Src {
        const uint16_t *w[INSTR];   // weight rows (instructions over token rows: unused)
        int tok[INSTR];             // token rows: the sorted index
        int kbeg, kend, nsteps;
    };

    // this lane's source rows: instruction j covers tile rows (wave*INSTR + j)*8 .. +8
    // (every instruction's 8 rows lie on one side of BT, a multiple of 16)
    __device__ __forceinline__ static Src sources(const ShrinkArgs &a, const TileRef &tr, int rb, int kbeg,
                                                  int kend) {
        Src sr;
        const int lane = lane_id(), wave = wave_id();
#pragma unroll
        for (int j = 0; j < INSTR; ++j) {
            const int r = (wave * INSTR + j) * 8 + (lane >> 3);
            if (r < BT) {
                int p = tr.tile * BT + r;
                p = p < tr.seg_count ? p : tr.seg_count - 1;
                sr.tok[j] = a.meta.sorted[tr.seg_start + p];
                sr.w[j] = a.x;
            } else {
                int row = rb * BR + (r - BT);
                row = row < a.rows ? row : a.rows - 1;
                const int i = row / a.rank, jr = row - i * a.rank;
                sr.tok[j] = 0;
                sr.w[j] = select_slice(a.a, i) + ((int64_t)tr.lora_id * a.rank + jr) * a.hidden;
            }
        }
        sr.kbeg = kbeg;
        sr.kend = kend;
        sr.nsteps = (kend - kbeg + 63) / 64;
        return sr;
    }

    // every instruction's 8 rows start at a multiple of 8, so the lane's row
    // index mod 8 and with it its global chunk (landing in slot lane & 7)
    // are the same for all of them
    __device__ __forceinline__ static int chunk_k() {
        const int lane = lane_id();
        return 8 * ((lane & 7) ^ ((lane >> 3) & 7));
    }

    __device__ __forceinline__ static void issue(const Src &sr, const uint16_t *const (&src)[INSTR], int step,
                                                 int buf, Stage *stage) {
        const int wave = wave_id();
        const int sc = step < sr.nsteps ? step : sr.nsteps - 1;   // past the end: reload, never skip
        const int k = sr.kbeg + sc * 64 + chunk_k();
        const int off = k + 8 <= sr.kend ? k : 0;
#pragma unroll
        for (int j = 0; j < INSTR; ++j)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src[j] + off),
                                             reinterpret_cast<void *>(&stage[buf][(wave * INSTR + j) * 1024]), 16,
                                             0, 0);
    }

    // The row pointers (the first use of the sorted indices, whose loads are
    // waited for here), then the first STAGES steps.
    __device__ __forceinline__ static void prime(const ShrinkArgs &a, Src &sr, const uint16_t *(&src)[INSTR],
                                                 Stage *stage) {
        const int lane = lane_id(), wave = wave_id();
#pragma unroll
        for (int j = 0; j < INSTR; ++j) {
            asm volatile("" : "+v"(sr.tok[j]));
            const int r = (wave * INSTR + j) * 8 + (lane >> 3);
            const int t = (unsigned)sr.tok[j] < (unsigned)a.num_tokens ? sr.tok[j] : 0;
            src[j] = r < BT ? a.x + (int64_t)t * a.ldx : sr.w[j];
        }
#pragma unroll
        for (int st = 0; st < STAGES; ++st) issue(sr, src, st, st, stage);
    }

    // (The sums are returned by value: the loop then works on values of its
    // own, which keeps the accumulators in place across iterations.)
    __device__ __forceinline__ static Acc finish(const Src &sr, const uint16_t *const (&src)[INSTR], Stage *stage) {
        Acc out;
        floatx4 (&acc)[MT][NTW] = out.v;
        const int lane = lane_id(), wave = wave_id();
        const int wr = wave % WR, wc = wave / WR;
        const int n16 = lane & 15, g = lane >> 4;
        const int kbeg = sr.kbeg, kend = sr.kend, nsteps = sr.nsteps;

#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

        for (int s = 0; s < nsteps; ++s) {
            // step s has landed once only the STAGES - 1 steps after it are
            // outstanding; the barrier publishes it to every wave
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((STAGES - 1) * INSTR));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            const unsigned char *sb = stage[s % STAGES];
            const bool mask = s == nsteps - 1 && ((kend - kbeg) & 63) != 0;
            // the operands of both 32-wide halves of the step, read before the
            // first MFMA
            u32x4 xa[2][NTW], wa[2][MT];
            auto read_half = [&](int h, int q) {
                const int c = 2 * g + h;
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const int r = (wc * NTW + nt) * 16 + n16;
                    xa[q][nt] = lds_read16(sb + r * 128 + 16 * (c ^ (r & 7)));
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int r = BT + (wr * MT + mt) * 16 + n16;
                    wa[q][mt] = lds_read16(sb + r * 128 + 16 * (c ^ (r & 7)));
                }
            };
            auto wait_half = [&](int q) {
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) after_wait(xa[q][nt]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) after_wait(wa[q][mt]);
            };
            read_half(0, 0);
            read_half(1, 1);
            lds_wait();
            wait_half(0);
            wait_half(1);
            // every wave has read the stage: refill it with step s + STAGES
            // before the MFMAs, so that STAGES steps are in flight while
            // they run
            __builtin_amdgcn_s_barrier();
            issue(sr, src, s + STAGES, s % STAGES, stage);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = h;
                if (mask && kbeg + s * 64 + 8 * (2 * g + h) + 8 > kend) {
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) xa[q][nt] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) wa[q][mt] = u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        acc[mt][nt] = mfma16x16x32(as_bf16x8(wa[q][mt]), as_bf16x8(xa[q][nt]), acc[mt][nt]);
            }
        }
        // drain the dummy loads issued past the end before the stages are reused
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
        return out;
    }

    // One piece start to end: the tile `tr`, the weight rows of row block
    // `rb`, the K range [kbeg, kend).
    __device__ __forceinline__ static Acc run(const ShrinkArgs &a, const TileRef &tr, int rb, int kbeg, int kend,
                                              Stage *stage) {
        Src sr = sources(a, tr, rb, kbeg, kend);
        const uint16_t *src[INSTR];
        prime(a, sr, src, stage);
        return finish(sr, src, stage);
    }
};

// The units (tile, row block, K chunk) walked in XCD-chunked order
// (UnitWalker), each run by the piece runner S.
template <class S>
__device__ __forceinline__ void unit_walk(const ShrinkArgs &a, int *smem, int *s_wsum, typename S::Stage *stage) {
    const int nslots = a.meta.nslots;
    const int total = build_tile_table<kThreads>(a.meta, S::BT, smem, s_wsum);
    const bool atomic = a.k_splits > 1;

    const UnitWalker walk(total * a.row_blocks * a.k_splits);
    for (int jj = walk.first;; jj += walk.stride) {
        const int u = walk.unit(jj);
        if (u < 0) break;
        const int ks = u % a.k_splits;
        const int rest = u / a.k_splits;
        const int rb = rest % a.row_blocks;
        const TileRef tr = lookup_tile(smem, nslots, rest / a.row_blocks);
        const int kbeg = ks * a.k_chunk;
        const int kend = min(kbeg + a.k_chunk, a.hidden);
        const typename S::Acc acc = S::run(a, tr, rb, kbeg, kend, stage);
        S::store(a, tr, rb, acc.v, atomic);
    }
}

template <int NT, int MR, int WR, int STAGES>
__global__ __launch_bounds__(kThreads) void shrink_lds_kernel(ShrinkArgs a) {
    using S = Staged<NT, MR, WR, STAGES>;
    extern __shared__ int smem[];
    __shared__ int s_wsum[kThreads / kWave];
    __shared__ __attribute__((aligned(1024))) typename S::Stage stage[STAGES];
    unit_walk<S>(a, smem, s_wsum, stage);
}

// Stream-K form of the LDS-staged shrink.  The work is the list of (tile,
// 64-wide K step) pairs, tile-major.  Workgroups form groups of RB, one per
// row block of the layer's weight rows; the groups (G of them, about two
// workgroups per CU in all) take equal contiguous shares of the list, the
// shares in XCD order (workgroup b sits on XCD b % 8, so consecutive shares
// and the members of a group stay on one XCD).  The members of a group walk
// the same tiles and K steps at the same time, so each token row they share
// comes from HBM once and from that XCD's L2 for the others.  A share cuts
// at most its first and its last tile:
//  - the first tile of a share that starts inside the tile is a later part:
//    each member stores its sums in its own slot (device-scope stores, which
//    are performed at the device's point of coherence), and once they are
//    complete (s_waitcnt vmcnt(0), then a barrier) increments the counter of
//    the tile and row block;
//  - the part holding the tile's first K step is the last piece of its
//    share: it waits until the counter shows every later part, adds their
//    slots (device-scope loads) to its own sums and stores the tile, then
//    sets the counter back to zero for the next launch.
// A later part is always the first piece of its share and never waits, so
// the waits end whenever every workgroup runs; each share has the same
// number of K steps, so every CU finishes at about the same time whatever
// the number of tiles.  A wait that passes kSkSpinLimit polls sets
// LORA_ERR_SYNC and goes on (the result is then unspecified).
constexpr int kSkSpinLimit = 1 << 18;
// Cache policy of the slot accesses: device scope (sc1), the bits an
// agent-scope atomic load or store carries.
constexpr int kCpolDevice = 16;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

template <class S>
__device__ __forceinline__ void sk_walk(const ShrinkArgs &a, const SkArgs &sk, int *smem, int *s_wsum,
                                        typename S::Stage *stage) {
    const int nslots = a.meta.nslots;
    const int total = build_tile_table<kThreads>(a.meta, S::BT, smem, s_wsum);
    const int tid = threadIdx.x;
    const int RB = a.row_blocks;
    const int nsteps = (a.hidden + 63) / 64;
    const long W = (long)total * nsteps;
    // groups per XCD (the launcher makes it at least one); with fewer steps
    // than groups only the first W groups are used, so that every share in
    // use holds at least one step
    const int gx = (int)(gridDim.x / kNumXcd) / RB;
    const int i = (int)(blockIdx.x / kNumXcd);
    if (i >= gx * RB) return;
    const int gq = (int)(blockIdx.x % kNumXcd) * gx + i / RB, r = i % RB;
    const int G = W < (long)(kNumXcd * gx) ? (int)W : kNumXcd * gx;
    if (gq >= G) return;
    const long end = W * (gq + 1) / G;
    // the group whose share holds step `it` of the list
    auto owner = [&](long it) { return (int)(((it + 1) * G - 1) / W); };
    // member r of group k: its slot
    auto slot_rsrc = [&](int k) {
        return __builtin_amdgcn_make_buffer_rsrc(sk.slots + (long)(k * RB + r) * S::SLOT, 0, S::SLOT * 4, 0x00020000);
    };

    for (long cur = W * gq / G; cur < end;) {
        const int t = (int)(cur / nsteps);
        const int s0 = (int)(cur - (long)t * nsteps);
        const int s1 = (int)min((long)nsteps, (long)s0 + (end - cur));
        cur += s1 - s0;
        const TileRef tr = lookup_tile(smem, nslots, t);
        typename S::Acc res = S::run(a, tr, r, 64 * s0, min(64 * s1, a.hidden), stage);
        floatx4 (&acc)[S::MT][S::NTW] = res.v;
        if (s0 > 0 || s1 < nsteps) {
            const long first = (long)t * nsteps;
            const int ga = owner(first);
            int32_t *count = sk.counters + (ga + 1) * RB + r;   // the first share boundary inside the tile
            if (s0 > 0) {
                const __amdgpu_buffer_rsrc_t slot = slot_rsrc(gq);
#pragma unroll
                for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < S::NTW; ++nt)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, acc[mt][nt]), slot, 16 * tid,
                                                               (mt * S::NTW + nt) * 16 * kThreads, kCpolDevice);
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                __syncthreads();
                if (tid == 0) __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                continue;
            }
            const int gb = owner(first + nsteps - 1);
            if (tid == 0) {
                int n = 0;
                while (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < gb - gq &&
                       n < kSkSpinLimit) {
                    ++n;
                    __builtin_amdgcn_s_sleep(8);
                }
                if (n == kSkSpinLimit)
                    __hip_atomic_store(sk.status, (int)LORA_ERR_SYNC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(count, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            // the later parts' sums, up to 16 16-byte loads in flight at a time
            constexpr int P = S::MT * S::NTW;
            constexpr int B = P < 24 ? P : 24;
            for (int k = gq + 1; k <= gb; ++k) {
                const __amdgpu_buffer_rsrc_t slot = slot_rsrc(k);
#pragma unroll
                for (int p0 = 0; p0 < P; p0 += B) {
                    floatx4 v[B];
#pragma unroll
                    for (int q = 0; q < B; ++q)
                        if (p0 + q < P)
                            v[q] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                   slot, 16 * tid, (p0 + q) * 16 * kThreads, kCpolDevice));
#pragma unroll
                    for (int q = 0; q < B; ++q)
                        if (p0 + q < P) acc[(p0 + q) / S::NTW][(p0 + q) % S::NTW] += v[q];
                }
            }
        }
        S::store(a, tr, r, acc, false);
    }
}

template <int NT, int MR, int WR, int STAGES>
__global__ __launch_bounds__(kThreads) void shrink_sk_kernel(ShrinkArgs a, SkArgs sk) {
    using S = Staged<NT, MR, WR, STAGES>;
    extern __shared__ int smem[];
    __shared__ int s_wsum[kThreads / kWave];
    __shared__ __attribute__((aligned(1024))) typename S::Stage stage[STAGES];
    sk_walk<S>(a, sk, smem, s_wsum, stage);
}

// Rows of the batch's active tokens set to zero, ahead of a split-K shrink
// into a fresh buffer (its K chunks are added with atomics).  Rows of tokens
// with id -1 are not touched.  Units are 16-token tiles.
__global__ __launch_bounds__(kThreads) void zero_rows_kernel(ShrinkArgs a) {
    extern __shared__ int smem[];
    __shared__ int s_wsum[kThreads / kWave];
    const int nslots = a.meta.nslots;
    const int total = build_tile_table<kThreads>(a.meta, 16, smem, s_wsum);
    const int per_tok = a.rank / 4;              // 16-byte pieces per token row of a slice
    const int per_unit = 16 * a.rows / 4;
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
    const UnitWalker walk(total);
    for (int jj = walk.first;; jj += walk.stride) {
        const int u = walk.unit(jj);
        if (u < 0) break;
        const TileRef tr = lookup_tile(smem, nslots, u);
        for (int x = threadIdx.x; x < per_unit; x += kThreads) {
            const int prow = x / (a.rows / 4), rest = x % (a.rows / 4);
            const int i = rest / per_tok, piece = rest % per_tok;
            const int pp = tr.tile * 16 + prow;
            if (pp >= tr.seg_count) continue;
            const int t = a.meta.sorted[tr.seg_start + pp];
            if ((unsigned)t >= (unsigned)a.num_tokens) continue;
            *reinterpret_cast<floatx4 *>(a.buf + ((int64_t)i * a.num_tokens + t) * a.rank + 4 * piece) = z;
        }
    }
}

typedef void (*ShrinkFn)(ShrinkArgs);

template <int NT, int WK>
ShrinkFn pick_mt(int mt) {
    switch (mt) {
        case 1: return shrink_kernel<NT, 1, WK>;
        case 2: return shrink_kernel<NT, 2, WK>;
        case 3: return shrink_kernel<NT, 3, WK>;
        default: return shrink_kernel<NT, 4, WK>;
    }
}

template <int NT>
ShrinkFn pick_wk(int wk, int mt) {
    switch (wk) {
        case 1: return pick_mt<NT, 1>(mt);
        case 2: return pick_mt<NT, 2>(mt);
        default: return pick_mt<NT, 4>(mt);
    }
}

ShrinkFn pick(int nt, int wk, int mt) {
    switch (nt) {
        case 1: return pick_wk<1>(wk, mt);
        case 2: return pick_wk<2>(wk, mt);
        case 4: return pick_wk<4>(wk, mt);
        default: return pick_wk<8>(wk, mt);
    }
}


// LDS-staged configurations: tokens x rows per workgroup, wave layout, stages.
typedef void (*SkFn)(ShrinkArgs, SkArgs);
struct StagedCfg {
    int nt, mr, wr, stages;
    bool automatic;   // eligible for the automatic choice
    ShrinkFn fn;
    SkFn sk;          // the same tile in the stream-K kernel
};
const StagedCfg kStaged[] = {
    {4, 12, 4, 3, true, shrink_lds_kernel<4, 12, 4, 3>, shrink_sk_kernel<4, 12, 4, 3>},    // 0: 64 tokens x 192 rows
    {8, 12, 4, 3, false, shrink_lds_kernel<8, 12, 4, 3>, shrink_sk_kernel<8, 12, 4, 3>},   // 1: 128 x 192 (one wave per SIMD: slow)
    {4, 8, 4, 4, true, shrink_lds_kernel<4, 8, 4, 4>, shrink_sk_kernel<4, 8, 4, 4>},      // 2: 64 x 128
    {4, 4, 4, 4, true, shrink_lds_kernel<4, 4, 4, 4>, shrink_sk_kernel<4, 4, 4, 4>},      // 3: 64 x 64
    {4, 2, 2, 4, true, shrink_lds_kernel<4, 2, 2, 4>, shrink_sk_kernel<4, 2, 2, 4>},      // 4: 64 x 32
    {2, 12, 4, 4, true, shrink_lds_kernel<2, 12, 4, 4>, shrink_sk_kernel<2, 12, 4, 4>},    // 5: 32 x 192
    {8, 4, 4, 4, true, shrink_lds_kernel<8, 4, 4, 4>, shrink_sk_kernel<8, 4, 4, 4>},      // 6: 128 x 64
    {8, 2, 2, 4, true, shrink_lds_kernel<8, 2, 2, 4>, shrink_sk_kernel<8, 2, 2, 4>},      // 7: 128 x 32
    {2, 4, 4, 4, true, shrink_lds_kernel<2, 4, 4, 4>, shrink_sk_kernel<2, 4, 4, 4>},      // 8: 32 x 64
    {2, 2, 2, 4, true, shrink_lds_kernel<2, 2, 2, 4>, shrink_sk_kernel<2, 2, 2, 4>},      // 9: 32 x 32
    {4, 6, 2, 5, true, shrink_lds_kernel<4, 6, 2, 5>, shrink_sk_kernel<4, 6, 2, 5>},      // 10: 64 x 96
    {8, 6, 2, 4, true, shrink_lds_kernel<8, 6, 2, 4>, shrink_sk_kernel<8, 6, 2, 4>},      // 11: 128 x 96
    {8, 8, 4, 4, false, shrink_lds_kernel<8, 8, 4, 4>, shrink_sk_kernel<8, 8, 4, 4>},     // 12: 128 x 128, 4 stages (one per CU)
    {8, 8, 4, 2, true, shrink_lds_kernel<8, 8, 4, 2>, shrink_sk_kernel<8, 8, 4, 2>},      // 13: 128 x 128, 2 stages (two per CU)
    {4, 6, 2, 3, false, shrink_lds_kernel<4, 6, 2, 3>, shrink_sk_kernel<4, 6, 2, 3>},     // 14: 64 x 96, 3 stages (two per CU)
    {4, 6, 2, 7, false, shrink_lds_kernel<4, 6, 2, 7>, shrink_sk_kernel<4, 6, 2, 7>},     // 15: 64 x 96, 7 stages
    {2, 4, 4, 10, false, shrink_lds_kernel<2, 4, 4, 10>, shrink_sk_kernel<2, 4, 4, 10>},   // 16: 32 x 64, 10 stages
    {4, 4, 4, 8, false, shrink_lds_kernel<4, 4, 4, 8>, shrink_sk_kernel<4, 4, 4, 8>},     // 17: 64 x 64, 8 stages
    {2, 2, 2, 12, false, shrink_lds_kernel<2, 2, 2, 12>, shrink_sk_kernel<2, 2, 2, 12>},   // 18: 32 x 32, 12 stages
};
constexpr int kNumStaged = sizeof(kStaged) / sizeof(kStaged[0]);

constexpr int kStagedGridCap = 512;   // workgroups of the staged unit walk, at most
constexpr int kSkMinSteps = 8;   // K steps per workgroup share, at least
constexpr int kSkBigCfg = 1;     // the 128 x 192 tile
constexpr long kSkBigShare = 64; // K steps per CU from which it is taken

}  // namespace

// Tile selection from host-known sizes only (no device sync).  The expected
// segment length N / min(N, max_loras + 1) picks the kernel: short segments
// (decode-like) use the direct-load kernel with K interleaved over the waves,
// long ones the LDS-staged kernel with a tile of 64-128 tokens x up to 192
// rows.  K chunks (combined with float atomics) are added only when the units
// would not cover the GPU.  `cfg` fields > 0 override the choice (tuning).
namespace {

struct ShrinkPlan {
    bool staged;
    bool sk;          // stream-K (sk_fn)
    ShrinkFn fn;
    SkFn sk_fn;
    long slot_floats; // stream-K: floats of one part slot
    int tile_tokens, row_blocks, k_splits, k_chunk;
    long units_upper;
};

ShrinkPlan plan_shrink(int n, int nslots, int rows, int hidden, const ShrinkTuning &cfg) {
    ShrinkPlan pl;
    const int mtiles = (rows + 15) / 16;
    const int segs = nslots < n ? nslots : n;
    const int avg = (n + segs - 1) / segs;
    const int max_ks = (hidden + 255) / 256;

    pl.staged = cfg.variant == 3 || (cfg.variant == 0 && avg >= 24);
    pl.sk = false;
    int rows_per_wg;
    int idx = -1;
    int forced_ks = cfg.k_splits;
    int model_ks = 1;
    if (pl.staged) {
        idx = cfg.staged_cfg;
        if (idx <= 0 || idx > kNumStaged) {
            // Cost model: a unit streams (tokens + rows) x K_chunk bf16 through
            // LDS at about the same rate on every CU, so the time goes as
            // max(units / CUs, 1) x bytes per unit; every extra K chunk adds
            // one float atomic per active (token, row) element.
            const double cus = 256.0, bytes_per_atomic = 100.0;   // fitted to measured split-K cost
            double best = 1e300;
            for (int c = 0; c < kNumStaged; ++c) {
                if (!kStaged[c].automatic) continue;
                const int T = 16 * kStaged[c].nt, R = 16 * kStaged[c].mr;
                const double tiles = (double)segs * ((avg + T - 1) / T);
                const double rb = (rows + R - 1) / R;
                for (int ksc = 1; ksc <= 4; ksc *= 2) {
                    if (forced_ks > 0 && ksc != forced_ks) continue;
                    const double units = tiles * rb * ksc;
                    const double per_unit = (double)(T + R) * 2.0 * ((hidden + ksc - 1) / ksc);
                    double cost = (units / cus > 1.0 ? units / cus : 1.0) * per_unit;
                    // waste on rows past S*r and tokens past the segment end
                    cost *= (rb * R) / (double)rows;
                    if (ksc > 1) cost += ksc * (double)n * rows * bytes_per_atomic / cus;
                    if (cost < best) {
                        best = cost;
                        idx = c;
                        model_ks = ksc;
                    }
                }
            }
            if (forced_ks <= 0) forced_ks = model_ks;
        } else {
            idx -= 1;
        }
        const StagedCfg &c = kStaged[idx];
        pl.tile_tokens = 16 * c.nt;
        rows_per_wg = 16 * c.mr;
        pl.fn = c.fn;
    } else {
        int nt = cfg.tile_tokens > 0 ? cfg.tile_tokens / 16 : (avg <= 16 ? 1 : (avg <= 32 ? 2 : 4));
        if (nt != 1 && nt != 2 && nt != 4) nt = 8;
        int wk = cfg.waves_k;
        if (wk != 1 && wk != 2 && wk != 4) wk = mtiles >= 8 ? 1 : (mtiles >= 4 ? 2 : 4);
        const int wr = 4 / wk;
        int mt = cfg.mtiles_per_wave > 0 ? cfg.mtiles_per_wave : (mtiles + wr - 1) / wr;
        if (mt > 4) mt = 4;
        if (nt == 8 && mt > 2) mt = 2;
        pl.tile_tokens = 16 * nt;
        rows_per_wg = wr * mt * 16;
        pl.fn = pick(nt, wk, mt);
    }
    pl.row_blocks = (rows + rows_per_wg - 1) / rows_per_wg;

    int tiles_upper = (n + pl.tile_tokens - 1) / pl.tile_tokens + segs;
    const int busy = ((n + pl.tile_tokens - 1) / pl.tile_tokens + (segs + 1) / 2) * pl.row_blocks;
    int ks = 1;
    if (!pl.staged && busy < 256) ks = (256 + busy - 1) / busy;
    if (forced_ks > 0) ks = forced_ks;
    if (ks > max_ks) ks = max_ks;
    if (ks < 1) ks = 1;
    int chunk = (hidden + ks - 1) / ks;
    chunk = (chunk + 63) / 64 * 64;
    ks = (hidden + chunk - 1) / chunk;
    pl.k_splits = ks;
    pl.k_chunk = chunk;
    pl.units_upper = (long)tiles_upper * pl.row_blocks * ks;

    // Stream-K for every staged batch of at least kSkMinTokens tokens (whose
    // library-owned area holds the part slots): its equal shares leave no CU
    // with a unit more than another, and a K split needs no float atomics
    // into a cleared buffer (the slots combine the parts).  The unit walk
    // stays for smaller batches.  LORA_SHRINK_SK=2 forces it for any staged
    // batch that size, LORA_SHRINK_SK=1 turns it off.
    const bool automatic = cfg.stream_k == 0 && cfg.k_splits <= 0 && cfg.variant == 0 && cfg.staged_cfg <= 0;
    bool sk_auto = automatic;
    // Long K walks over more than 128 weight rows (the large shape): the
    // 128 x 192 tile as stream-K, one workgroup per CU, reads each token row
    // once per 192 rows instead of once per 128, and its shares are long
    // enough (at least kSkBigShare steps per CU) to carry the one-deep
    // occupancy.  On shorter walks (prefill) it loses to the tile the cost
    // model picks.
    if (automatic && pl.staged && n >= kSkMinTokens && rows > 128) {
        const StagedCfg &big = kStaged[kSkBigCfg];
        const long tiles = (n + 16 * big.nt - 1) / (16 * big.nt) + segs;
        const long rbs = (rows + 16 * big.mr - 1) / (16 * big.mr);
        if (tiles * rbs * ((hidden + 63) / 64) >= 256L * kSkBigShare) {
            idx = kSkBigCfg;
            pl.tile_tokens = 16 * big.nt;
            pl.row_blocks = (int)rbs;
            tiles_upper = (int)tiles;
        }
    }
    if (pl.staged && n >= kSkMinTokens && (cfg.stream_k == 2 || sk_auto)) {
        const StagedCfg &c = kStaged[idx];
        pl.sk = true;
        pl.fn = nullptr;
        pl.sk_fn = c.sk;
        pl.slot_floats = 256 * c.nt * c.mr;
        pl.k_splits = 1;
        pl.k_chunk = (hidden + 63) / 64 * 64;
        // K steps of the list, at most
        pl.units_upper = (long)tiles_upper * ((hidden + 63) / 64);
    }
    return pl;
}

}  // namespace

int shrink_launches(int n, int nslots, int rows, int hidden, bool overwrite, const ShrinkTuning &cfg) {
    if (n < 1) return 0;
    const ShrinkPlan pl = plan_shrink(n, nslots, rows, hidden, cfg);
    return (overwrite && !pl.sk && pl.k_splits > 1) ? 2 : 1;
}

hipError_t launch_shrink(const ShrinkArgs &in, const SkArgs &sk, const ShrinkTuning &cfg, hipStream_t s) {
    ShrinkArgs a = in;
    const int n = a.num_tokens;
    const int nslots = a.meta.nslots;
    ShrinkPlan pl = plan_shrink(n, nslots, a.rows, a.hidden, cfg);
    if (pl.sk && (!sk.slots || !sk.counters || !sk.status)) {
        // the area has no stream-K part (cannot happen for a batch of this
        // size, which the region was bound for): the unit-walking kernel
        ShrinkTuning c = cfg;
        c.stream_k = 1;
        pl = plan_shrink(n, nslots, a.rows, a.hidden, c);
    }
    if (pl.sk) {
        a.row_blocks = pl.row_blocks;
        a.k_splits = 1;
        a.k_chunk = pl.k_chunk;
        a.num_units = 0;
        a.meta.lds_tokens = 0;
        const size_t lds = sizeof(int) * (size_t)(4 * nslots + 1);
        const int rb = pl.row_blocks;
        long grid = resident_grid(reinterpret_cast<const void *>(pl.sk_fn), kThreads, lds);
        if (grid > kSkMaxGroups) grid = kSkMaxGroups;
        if (grid > kSkSlotArea / pl.slot_floats) grid = kSkSlotArea / pl.slot_floats;
        if (cfg.grid_cap > 0) {
            if (grid > cfg.grid_cap) grid = cfg.grid_cap;   // tuning and tests: exactly this many
        } else {
            const long by_work = pl.units_upper * rb / kSkMinSteps;
            if (grid > by_work) grid = by_work;
        }
        // whole groups of rb workgroups on every XCD, and a counter per
        // share boundary and row block
        long gx = grid / kNumXcd / rb;
        if ((kNumXcd * gx + 1) * rb > kSkCounterWords) gx = (kSkCounterWords / rb - 1) / kNumXcd;
        if (gx >= 1) {
            hipLaunchKernelGGL(pl.sk_fn, dim3((unsigned)(kNumXcd * gx * rb)), dim3(kThreads), lds, s, a, sk);
            return hipGetLastError();
        }
        ShrinkTuning c = cfg;   // too many row blocks for the resident workgroups: walk units
        c.stream_k = 1;
        pl = plan_shrink(n, nslots, a.rows, a.hidden, c);
    }
    a.row_blocks = pl.row_blocks;
    a.k_splits = pl.k_splits;
    a.k_chunk = pl.k_chunk;
    a.num_units = (int)pl.units_upper;

    if (a.overwrite && a.k_splits > 1) {
        // a fresh buffer combined from K chunks with atomics: zero its rows first
        ShrinkArgs z = a;
        z.meta.lds_tokens = 0;
        const size_t zlds = sizeof(int) * (size_t)(4 * nslots + 1);
        const long zunits = (n + 15) / 16 + (nslots < n ? nslots : n);
        const long zgrid = persistent_grid(zunits, 1024, reinterpret_cast<const void *>(zero_rows_kernel), kThreads,
                                           zlds);
        hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)zgrid), dim3(kThreads), zlds, s, z);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    // small batches: the direct-load kernel keeps the sorted indices in LDS
    a.meta.lds_tokens = (!pl.staged && n <= kLdsTokensMax) ? n : 0;
    const size_t lds = sizeof(int) * (size_t)(4 * nslots + 1 + a.meta.lds_tokens);
    const long grid = persistent_grid(pl.units_upper, cfg.grid_cap > 0 ? cfg.grid_cap : (pl.staged ? kStagedGridCap : 1024),
                                      reinterpret_cast<const void *>(pl.fn), kThreads, lds);
    hipLaunchKernelGGL(pl.fn, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace lora
