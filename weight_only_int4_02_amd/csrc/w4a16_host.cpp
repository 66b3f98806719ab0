// Pure host logic of libw4a16: argument checks, workspace sizing, the choice of
// kernel and split, status strings.  No HIP call is made here, so every error
// path can be exercised on a machine without a GPU.
//
// The error convention follows torchchat issue "linear:int4 quantization
// regression testing": a weight whose K is not a multiple of the group size is
// refused with an explicit status (never skipped silently) unless the caller
// asks for a partial last group (option 2 of that discussion).
#include <stdint.h>
#include <string.h>

#include "w4a16.h"
#include "w4a16_internal.hpp"

namespace w4a16 {

Geom make_geom(int64_t M, int64_t N, int64_t K, int32_t g, uint32_t flags) {
    Geom geo;
    geo.M = M;
    geo.N = N;
    geo.K = K;
    geo.g = g;
    geo.NT = (N + 15) / 16;
    geo.KT = (K + 127) / 128;
    geo.G = (K + g - 1) / g;
    geo.GW = (geo.G + 7) / 8;
    geo.sym = (flags & W4A16_SYMMETRIC) != 0;
    geo.bf16 = (flags & W4A16_BF16) != 0;
    return geo;
}

// Kernel choice and its shape parameters, from sweeps on MI355X over the
// Llama-2 7B / 70B linear shapes.
//
// Small-M path (M <= 64, or forced): NB weight tiles per workgroup trade
// activation reuse (activation bytes per weight byte are M / (4 NB)) against
// the number of workgroups; few waves per workgroup once the activation
// fragments take many registers (M > 8); a ring of 2 register stages, 4 when
// a wave's stage is a single tile (NB = 1, M > 8).
//
// Large-M path: the largest output tile that still gives every compute unit
// a workgroup (256 CUs).
GemmPlan plan_gemm(const Geom &geo, uint32_t flags) {
    GemmPlan p;
    bool small;
    if (flags & W4A16_PATH_SMALL_M)
        small = true;
    else if (flags & W4A16_PATH_LARGE_M)
        small = false;
    else
        small = geo.M <= kSmallMMax ||
                (geo.M <= kSmallMMaxNarrow && geo.NT <= 256) ||
                (geo.M <= kSmallMMaxNarrowShortK && geo.NT <= 256 && geo.KT <= 32 && !geo.bf16 &&
                 geo.g >= 128);
    p.path = small ? PATH_SMALL : PATH_LARGE;
    p.ws_bytes = 0;
    p.splits = 1;
    // Small-M kernel shape, from measured sweeps over the Llama-2 7B / 70B
    // shapes (g = 128, M = 1..32).  Few output rows (N <= 4096) need the K
    // split across many waves; long K (>= 16384) prefers few waves with deep
    // rings; from M = 16 on, four weight tiles share each activation fragment
    // and, where that leaves fewer than 256 workgroups, K is also split
    // across workgroups (fp32 partial sums + a reduce kernel).
    // two activation tiles per workgroup above M = 16, except M <= 32 with at
    // most 256 weight tiles, where two workgroups per weight block (and a K
    // split) fill the chip better
    p.mtiles = (geo.M > 16 && !(geo.M <= 32 && geo.NT <= 256)) ? 2 : 1;
    const int64_t mblocks = (geo.M + 16 * p.mtiles - 1) / (16 * p.mtiles);
    if (geo.M <= 8 || (geo.M <= 16 && geo.NT <= 256 && geo.KT <= 32)) {
        if (geo.NT <= 256) {
            const bool wide = geo.M == 1 && geo.KT <= 32;
            p.waves = wide ? 8 : 4;
            p.nb = 1;
            p.depth = wide ? 2 : 4;
        } else if (geo.NT <= 1024) {
            const bool long_k = geo.KT >= 128;
            p.waves = long_k ? 4 : 16;
            p.nb = long_k ? 2 : 4;
            p.depth = long_k ? 3 : 2;
        } else if (geo.M <= 4 || geo.NT <= 2048) {
            p.waves = 8;
            p.nb = 2;
            p.depth = 3;
        } else {
            p.waves = 4;
            p.nb = 4;
            p.depth = 2;
        }
    } else {
        // eight weight tiles share each activation fragment at M = 17..32
        // over many weight tiles (fp16, g >= 128): half the activation
        // re-reads of four
        const bool wide_nb = geo.M > 16 && geo.M <= 32 && geo.NT >= 1024 && !geo.bf16 && geo.g >= 128;
        p.nb = wide_nb ? 8 : 4;
        // At M = 33..64 (two activation tiles per workgroup), eight weight
        // tiles where four would make 257..511 workgroups, which the rule
        // below turns into a two-way K split and a reduce launch: eight make
        // at most 256 and no split, and read the activations half as often
        // (Llama-2 7B qkv at M = 64 22.9 -> 19.7 us, M = 48 20.5 -> 18.7 us;
        // o_proj, gate+up and down stay at four, where eight was 20-33 %
        // slower)
        if (geo.M > 32 && geo.M <= 64 && !geo.bf16 && geo.g >= 128) {
            const int64_t wgs4 = ((geo.NT + 3) / 4) * mblocks;
            if (wgs4 > 256 && wgs4 < 512)
                p.nb = 8;
        }
        // eight waves over at most 256 weight tiles (they then take the
        // activation stages through LDS, below): with four, down (K = 11008)
        // at M = 48..128 ran one 4-wave workgroup per compute unit; eight
        // were 12-20 % faster there (M = 64 20.0 -> 17.7 us, M = 96 28.0 ->
        // 22.6), and level at M = 17..32
        p.waves = (geo.NT <= 256 && geo.M > 16 && p.nb != 8) ? 8 : 4;
        p.depth = 2;
        const int64_t wgs = ((geo.NT + p.nb - 1) / p.nb) * mblocks;
        while (2 * p.splits * wgs <= 256 && 2 * p.splits <= geo.KT)
            p.splits *= 2;
        if (p.splits == 1 && geo.M > 16 && wgs > 256 && wgs < 512 && geo.KT >= 32)
            p.splits = 2;
    }
    // Balance over the 256 compute units (fp16, g >= 128, M = 5..32, K up to
    // 8192): where one workgroup per compute unit takes 3 or 6 weight tiles
    // (5 or 6 for the 6-tile shape), use exactly that and no split.  With 4
    // or 8 tiles per workgroup the busiest units did up to 1.5x the average
    // (gate+up 22016 x 4096: 8 tiles against 5.4): M = 16 15.7 -> 12.5 us,
    // M = 32 19.6 -> 15.6 us; qkv 12288 x 4096 M = 8..32 0.6-1.0 us faster.
    const int jpg = geo.g >= 128 ? 4 : (int)(geo.g / 32);
    if (!geo.bf16 && jpg == 4 && geo.M > 4 && geo.M <= 32 && geo.KT <= 64) {
        for (int mt = 1; mt <= (geo.M > 16 ? 2 : 1); mt++) {
            const int64_t mb = (geo.M + 16 * mt - 1) / (16 * mt);
            const int64_t need = (geo.NT * mb + 255) / 256;
            const int nb = need == 3 ? 3 : (need == 5 || need == 6) ? 6 : 0;
            if (nb && small_shape_fits(jpg, geo.bf16, 4, nb, mt)) {
                p.nb = nb;
                p.mtiles = mt;
                p.waves = 4;
                p.depth = 2;
                p.splits = 1;
                break;
            }
        }
    }
    const int small_splits = p.splits;

    // Large-M kernel, from measured sweeps (Llama-2 7B shapes, M = 64..2048):
    // 32 x 256 output tiles (4 compute waves) when 128 x 256 tiles would be
    // fewer than 32 (or M <= 64); 128 x 256 tiles (8 compute waves) from 128
    // of them on; 128 x 128 tiles (4 compute waves) in between, where they
    // spread the work over more workgroups.  K is split across workgroups
    // until the workgroups would outnumber the 256 CUs or a slice would drop
    // below four 128-column tiles.
    const int64_t t3 = ((geo.M + 127) / 128) * ((geo.N + 255) / 256);
    const bool narrow = geo.M <= 64 || t3 < 32;
    // The 128 x 256 tile is four 128 x 64 compute waves for g >= 128 (each
    // dequantized weight fragment feeds eight MFMAs: half the dequantization
    // per MFMA of eight 64 x 64 waves; Llama-2 7B at M = 2048 on the same
    // box: fp16 3-6 % faster, bf16 17-23 %), eight 64 x 64 waves otherwise.
    const bool tall = geo.g >= 128;
    // and 128 x 256 tiles from 32 of them on (g >= 128) where the K split
    // that fills the chip still leaves each workgroup at least 16 stages:
    // its four 128 x 64 waves dequantize half as much per MFMA as the 64 x 64
    // waves of the 128 x 128 tile (Llama-2 7B down at M = 384, 512 8 %
    // faster, 70B down at M = 256 150 -> 127 us, 70B o_proj at M = 256 5 %;
    // o_proj at M = 512, 8 stages per workgroup, was 5 % slower)
    int64_t s3 = 1;
    while (t3 * s3 * 2 <= 256 && geo.KT / (s3 * 2) >= 4)
        s3 *= 2;
    const bool long_slices = tall && t3 >= 32 && geo.KT / s3 >= 16;
    p.large_shape = narrow ? 7 : (t3 >= 128 || long_slices) ? (tall ? 12 : 3) : 0;
    // 256 x 256 tiles (eight 128 x 64 waves, two per SIMD: 6-12 % faster per
    // tile on the same box) where their rounds over the 256 CUs are used at
    // least as well as those of the 128 x 256 tiles, counting that gain:
    // Llama-2 7B gate+up at M = 512 (172 tiles against 344) and M = 2048
    // (688 against 1376); not where half the CUs would idle (o_proj, down at
    // M = 2048) or a half round would be added (qkv at M = 2048).
    const int64_t t4 = ((geo.M + 255) / 256) * ((geo.N + 255) / 256);
    auto round_use = [](int64_t t) { return (double)t / (256.0 * (double)((t + 255) / 256)); };
    if (p.large_shape == 12 && geo.M >= 256 && round_use(t4) * 1.06 > round_use(t3))
        p.large_shape = 14;
    // 128 x 192 tiles (four 128 x 48 waves) where their rounds over the CUs
    // are used clearly better than the chosen shape's, both with their K
    // splits: qkv and gate+up at M = 128..512 (4-10 % faster on one box),
    // where 256-column tiles leave a quarter to a third of a round idle
    auto splits_for = [&](int64_t t) {
        int s = 1;
        while (t * s * 2 <= 256 && geo.KT / (s * 2) >= 4)
            s *= 2;
        return s;
    };
    const int64_t t17 = ((geo.M + 127) / 128) * ((geo.N + 191) / 192);
    {
        const int64_t tc = narrow ? ((geo.M + 31) / 32) * ((geo.N + 255) / 256)
                           : p.large_shape == 14 ? t4
                           : p.large_shape == 3 || p.large_shape == 12 ? t3
                                                : ((geo.M + 127) / 128) * ((geo.N + 127) / 128);
        if (geo.g >= 128 && !narrow &&
            round_use(t17 * splits_for(t17)) > 1.15 * round_use(tc * splits_for(tc)))
            p.large_shape = 17;
    }
    // The 128 x 128 tile from four 128 x 32 waves (g >= 128) rather than
    // four 64 x 64 ones: half the dequantization per MFMA for twice the
    // activation reads from LDS.  Same box, A-B-A-B: Llama-2 7B down M = 256
    // 43.5 -> 37.9 us, o_proj M = 512 31.8 -> 29.3, down M = 512 59.5 ->
    // 57.4; 70B o_proj M = 128 34.6 -> 31.7.  bf16 (with the 128 x 192
    // tile, two A-B pairs of the prefill bench): prefill7b bf16 828 -> 867
    // TFLOP/s (qkv M = 128 37.9 -> 26.9 us, down M = 256 50.2 -> 36.9,
    // o_proj M = 512 40.0 -> 29.9).
    if (p.large_shape == 0 && tall)
        p.large_shape = 18;
    // Wide tiles of eight 128-row compute waves, two per SIMD, with the
    // compute waves issuing the copies between their MFMA groups (g >= 128):
    // 128 x 384 (128 x 48 waves, 56 KiB per stage) where, without
    // a K split, it takes clearly less time than the chosen 128 x 256,
    // 256 x 256 or 128 x 192 tiles, and 128 x 512 (128 x 64 waves, 64 KiB per
    // stage) in place of 256 x 256 (80 KiB per stage for the same work) where
    // it makes no more tiles.  A call's time is taken as its rounds over the
    // 256 CUs times a tile's time: 1.0, 1.8, 0.8 and 1.42 in units of a
    // 128 x 256 tile (fitted to same-box times of the Llama-2 7B and 70B
    // shapes; a K split of s divides a tile's time by s).  Measured, A-B-A-B
    // on one box, against 128 x 192 / 128 x 256 / 256 x 256: gate+up M = 512
    // 99.8 -> 90.0 us, qkv M = 1024 103.7 -> 88.7, 70B qkv M = 1024 174.0 ->
    // 156.3, qkv M = 2048 184.7 -> 174.5, gate+up M = 2048 (128 x 512)
    // 309.2 -> 305.1; slower where it would split K (qkv M = 512) or add a
    // round (gate+up M = 2048 at 128 x 384).  bf16, two A-B pairs of the
    // prefill bench: gate+up M = 512 128.1 -> 102.7 us, qkv M = 2048 224.9
    // -> 203.2, gate+up M = 2048 380.0 -> 371.3.
    const int64_t t20 = ((geo.M + 127) / 128) * ((geo.N + 383) / 384);
    const int64_t t21 = ((geo.M + 127) / 128) * ((geo.N + 511) / 512);
    if (tall && geo.M >= 256 && splits_for(t20) == 1 &&
        (p.large_shape == 12 || p.large_shape == 14 || p.large_shape == 17)) {
        auto cost = [&](int64_t t, double unit) {
            const int s = splits_for(t);
            return (double)((t * s + 255) / 256) * unit / s;
        };
        const double cur = p.large_shape == 12 ? cost(t3, 1.0)
                           : p.large_shape == 14 ? cost(t4, 1.8)
                                                 : cost(t17, 0.8);
        if (cost(t20, 1.42) < 0.97 * cur)
            p.large_shape = 20;
    }
    if (p.large_shape == 14 && tall && t21 <= t4)
        p.large_shape = 21;
    const int64_t ltiles = p.large_shape == 20 ? t20
                           : p.large_shape == 21 ? t21
                           : p.large_shape == 17 ? t17
                           : narrow ? ((geo.M + 31) / 32) * ((geo.N + 255) / 256)
                           : p.large_shape == 14 ? t4
                           : p.large_shape == 3 || p.large_shape == 12 ? t3
                                                : ((geo.M + 127) / 128) * ((geo.N + 127) / 128);
    int large_splits = 1;
    while (ltiles * large_splits * 2 <= 256 && geo.KT / (large_splits * 2) >= 4)
        large_splits *= 2;

    p.splits = small ? small_splits : large_splits;
    // fewer waves where the chosen shape would not fit in registers
    while (p.waves > 4 && !small_shape_fits(jpg, geo.bf16, p.waves, p.nb, p.mtiles))
        p.waves /= 2;
    // Decode sizes (no split): stage the activations and group
    // constants in LDS (measured gains of 4-15 % at M = 1, none at M = 2..4
    // below 1024 weight tiles) if they fit beside the cross-wave sum within
    // 96 KiB per workgroup.
    p.lds = 0;
    if (small && geo.M <= 4 && p.splits == 1) {
        auto fits = [&](int waves, int nb) {
            return small_lds_bytes(geo.M, geo.K, geo.G, geo.GW, nb, geo.sym) +
                       (size_t)waves * nb * 1024 <= 96 * 1024;
        };
        if (geo.M == 1) {
            for (int waves : {8, 4})
                if (!p.lds && fits(waves, 1)) {
                    p.lds = 1;
                    p.waves = waves;
                    p.nb = 1;
                    p.depth = 3;
                }
        } else if (geo.NT > 1024 && fits(8, 2)) {
            p.lds = 1;
            p.waves = 8;
            p.nb = 2;
            p.depth = 2;
        }
    }
    // Activation stages through LDS (the XL form of the small-M kernel)
    // where the kernel is bound by the texture unit's cache-line lookups for
    // the activation fragments (g >= 128, M > 16): eight waves of four
    // weight tiles, and four waves of four tiles at two activation tiles
    // over many weight tiles.  Measured on MI355X: Llama-2 7B o_proj M = 32
    // 8.3 -> 8.0 us, M = 64 10.5 -> 9.5, M = 128 11.5 -> 9.9; gate+up M = 64
    // 31.6 -> 28.9.  The other shapes lost 1-12 % to the extra trip through
    // LDS (decode sizes, qkv, down with K = 11008).  bf16 (narrow weights on
    // the small-M kernel to M = 128 too): o_proj M = 128 20.8 -> 12.4 us,
    // down 42.2 -> 27.8 against the large-M kernel, gate+up M = 32 26.2 ->
    // 23.1, M = 64 36.0 -> 33.1.
    p.xl = 0;
    if (small && jpg == 4 && geo.M > 16 && p.nb == 4 && p.depth == 2 && !p.lds &&
        ((p.waves == 8 && p.mtiles <= 2) || (p.waves == 4 && p.mtiles == 2 && geo.NT >= 1024)))
        p.xl = 1;
    // Four waves of six weight tiles at one activation tile (the balance
    // shape of qkv-like weights at M = 17..32) and of eight tiles at two
    // activation tiles above M = 32: eight waves instead, taking the
    // activation stages through LDS (qkv M = 17..32 12.8 -> 11.8-12.2 us,
    // M = 48..64 19.0 -> 17.8; 70B qkv M = 32 22.8 -> 21.4, M = 64 32.0 ->
    // 30.2).  gate+up's six tiles at two activation tiles stay as they are
    // (2-3 % slower so), and so do eight tiles at M <= 32 (level).
    if (small && !geo.bf16 && jpg == 4 && geo.M > 16 && p.depth == 2 && !p.lds && p.waves == 4 &&
        ((p.nb == 6 && p.mtiles == 1) || (p.nb == 8 && p.mtiles == 2 && geo.M > 32))) {
        p.waves = 8;
        p.xl = 1;
    }
    // Narrow weights at M = 129..384 on the small-M kernel (eight waves of
    // four weight tiles at two activation tiles, activation stages through
    // LDS): eight weight tiles and no K split where that fits the call in
    // one round of 256 workgroups and four tiles do not (which split K two
    // ways up to 511 workgroups).  Same box: Llama-2 7B o_proj M = 192 20.7
    // -> 16.4 us, M = 256 18.7 -> 17.2; four stay ahead at M = 128 (one
    // round already) and M = 384 (eight would still take 1.5 rounds).
    if (small && !geo.bf16 && jpg == 4 && geo.M > 128 && p.xl && p.waves == 8 && p.nb == 4 &&
        p.mtiles == 2) {
        const int64_t mbl = (geo.M + 31) / 32;
        if (((geo.NT + 3) / 4) * mbl > 256 && ((geo.NT + 7) / 8) * mbl <= 256) {
            p.nb = 8;
            p.splits = 1;
        }
    }
    // Narrow weights (at most 256 row tiles) at M = 17..64 (g >= 128):
    // two weight tiles per workgroup over eight waves, activation stages
    // through LDS, and no K split where that still makes about 256
    // workgroups (no reduce launch).  Same box, A-B-A-B: Llama-2 7B o_proj
    // M = 32 7.9 -> 5.6 us, M = 48 9.3 -> 6.9, M = 64 9.5 -> 7.0; down
    // (K = 11008) M = 32 13.9 -> 12.8, M = 64 level.
    if (small && jpg == 4 && geo.M > 16 && geo.M <= 64 && geo.NT <= 256) {
        const int mt = geo.M > 32 ? 2 : 1;
        const int64_t mbl = (geo.M + 16 * mt - 1) / (16 * mt);
        if (((geo.NT + 1) / 2) * mbl >= 192) {
            p.waves = 8;
            p.nb = 2;
            p.mtiles = mt;
            p.depth = 2;
            p.splits = 1;
            p.xl = 1;
            p.lds = 0;
        }
    }
    // M = 5..16 (g >= 128, at least 192 row tiles): eight waves with
    // activation stages through LDS, one weight tile per workgroup up to 256
    // row tiles (no K split: 256 workgroups), two up to 512, three up to
    // 2048, four above; not for K > 16384 beyond 256 row tiles (70B down
    // was level to 4 % slower).  Same box, against the plan without it:
    // Llama-2 7B o_proj M = 8 5.2 -> 4.5 us, M = 16 6.5 -> 4.65; down M = 8
    // 10.3 -> 9.2, M = 16 11.06 -> 10.65 (no reduce launch); gate+up M = 8
    // 13.2 -> 12.3; 70B o_proj M = 8 13.2 -> 9.8, M = 16 12.9 -> 11.1, qkv
    // M = 16 14.5 -> 13.5, gate+up M = 16 61.7 -> 54.6.  bf16 (with the
    // rule below): decode7b bf16 2610 -> 2758 GB/s (o_proj M = 16 6.72 ->
    // 5.52 us, M = 32 8.6 -> 6.3, gate+up M = 16 15.8 -> 13.4).
    if (small && jpg == 4 && geo.M > 4 && geo.M <= 16 && geo.NT >= 192 &&
        (geo.NT <= 256 || geo.K <= 16384)) {
        const int nb = geo.NT <= 256 ? 1 : geo.NT <= 512 ? 2 : geo.NT <= 2048 ? 3 : 4;
        p.waves = 8;
        p.nb = nb;
        p.mtiles = 1;
        p.depth = 2;
        p.xl = 1;
        p.lds = 0;
        p.splits = 1;
        const int64_t wgs = (geo.NT + nb - 1) / nb;
        while (2 * p.splits * wgs <= 256 && 2 * p.splits <= geo.KT)
            p.splits *= 2;
    }
    // qkv-like weights (257..1024 row tiles) at M = 17..64 (g >= 128):
    // 32 activation rows per workgroup and three or six weight tiles, where
    // that makes 240..256 workgroups, over eight waves with activation stages
    // through LDS.  Same box: Llama-2 7B qkv M = 32 11.9 -> 10.6 us (three
    // tiles), M = 64 17.4 -> 15.5 (six); bf16 (three tiles only) qkv M = 32
    // 13.2 -> 11.6.
    // (bf16 also for wider weights up to M = 32: gate+up M = 17 21.6 ->
    // 19.6 us, M = 32 24.5 -> 21.4)
    if (small && jpg == 4 && geo.M > 16 && geo.M <= 64 && geo.NT > 256 &&
        (geo.NT <= 1024 || (geo.bf16 && geo.M <= 32))) {
        const int64_t mbl = (geo.M + 31) / 32;
        for (int nb : {3, 6}) {
            if (geo.bf16 && nb == 6)
                continue;  // (its bf16 instance would spill)
            const int64_t wgs = ((geo.NT + nb - 1) / nb) * mbl;
            // (bf16: three tiles whatever the count; at two rounds too, qkv
            // M = 48 26.2 -> 20.2 us, M = 64 27.5 -> 21.0, 70B qkv M = 64
            // 40.8 -> 35.6)
            if ((wgs >= 240 && wgs <= 256) || geo.bf16) {
                p.waves = 8;
                p.nb = nb;
                p.mtiles = 2;
                p.depth = 2;
                p.splits = 1;
                p.xl = 1;
                p.lds = 0;
                break;
            }
        }
    }
    if (p.splits > 1)
        p.ws_bytes = (size_t)p.splits * (size_t)geo.M * (size_t)geo.N * sizeof(float);
    return p;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static bool group_ok(int32_t g) { return g == 32 || g == 64 || g == 128 || g == 256; }

static int32_t check_flags(uint32_t flags, uint32_t allowed) {
    if (flags & ~allowed)
        return W4A16_ERR_FLAGS;
    if ((flags & W4A16_PATH_SMALL_M) && (flags & W4A16_PATH_LARGE_M))
        return W4A16_ERR_FLAGS;
    return W4A16_OK;
}

// Shape / group rules shared by repack, dequant and gemm.
static int32_t check_weight_shape(int64_t N, int64_t K, int32_t g, uint32_t flags) {
    if (N <= 0 || K <= 0 || (K % 8) != 0)
        return W4A16_ERR_SHAPE;
    // 32-bit offsets inside the kernels: every per-workgroup buffer slice (up
    // to 256 activation rows of K fp16 columns, 256 * K * 2 bytes) stays below
    // 2^31 bytes, so K < 2^22
    if (N > (int64_t(1) << 26) || K >= (int64_t(1) << 22) || N * K > (int64_t(1) << 34))
        return W4A16_ERR_SHAPE;
    if (!group_ok(g))
        return W4A16_ERR_GROUP;
    if ((K % g) != 0 && !(flags & W4A16_PARTIAL_LAST_GROUP))
        return W4A16_ERR_GROUP;
    return W4A16_OK;
}

}  // namespace w4a16

using namespace w4a16;

extern "C" {

const char *w4a16_status_str(int32_t status) {
    switch (status) {
    case W4A16_OK: return "W4A16_OK";
    case W4A16_ERR_NULL: return "W4A16_ERR_NULL: a required pointer is NULL";
    case W4A16_ERR_SHAPE: return "W4A16_ERR_SHAPE: bad M/N/K (must be > 0, K % 8 == 0, within limits)";
    case W4A16_ERR_GROUP: return "W4A16_ERR_GROUP: group size not in {32,64,128,256}, or K % g != 0 without W4A16_PARTIAL_LAST_GROUP";
    case W4A16_ERR_ALIGN: return "W4A16_ERR_ALIGN: a device pointer is not 16-byte aligned";
    case W4A16_ERR_WORKSPACE: return "W4A16_ERR_WORKSPACE: workspace too small";
    case W4A16_ERR_ARCH: return "W4A16_ERR_ARCH: the current device is not gfx950";
    case W4A16_ERR_HIP: return "W4A16_ERR_HIP: a HIP call failed";
    case W4A16_ERR_FLAGS: return "W4A16_ERR_FLAGS: unknown flag bits or conflicting path bits";
    default: return "unknown status";
    }
}

int32_t w4a16_check_pack_args(const uint8_t *codes, int64_t rows, int64_t cols,
                              const uint32_t *packed) {
    if (!codes || !packed)
        return W4A16_ERR_NULL;
    if (rows <= 0 || cols <= 0 || rows * cols > (int64_t(1) << 34))
        return W4A16_ERR_SHAPE;
    if (!aligned16(packed))
        return W4A16_ERR_ALIGN;
    return W4A16_OK;
}

int32_t w4a16_repack_size(int64_t N, int64_t K, int32_t g, uint32_t flags,
                          size_t *q_bytes, size_t *s_bytes, size_t *z_bytes) {
    if (!q_bytes || !s_bytes || !z_bytes)
        return W4A16_ERR_NULL;
    int32_t st = check_flags(flags, W4A16_SYMMETRIC | W4A16_PARTIAL_LAST_GROUP | W4A16_BF16);
    if (st)
        return st;
    st = check_weight_shape(N, K, g, flags);
    if (st)
        return st;
    Geom geo = make_geom(0, N, K, g, flags);
    *q_bytes = (size_t)(geo.NT * geo.KT * 1024);
    *s_bytes = (size_t)(geo.NT * geo.G * 16 * 2);
    *z_bytes = geo.sym ? 0 : (size_t)(geo.NT * geo.GW * 16 * 4);
    return W4A16_OK;
}

int32_t w4a16_check_repack_args(const uint32_t *qpacked, const uint16_t *scales,
                                const uint32_t *zeros, int64_t N, int64_t K,
                                int32_t g, uint32_t flags, const void *q_dev,
                                const void *s_dev, const void *z_dev) {
    int32_t st = check_flags(flags, W4A16_SYMMETRIC | W4A16_PARTIAL_LAST_GROUP | W4A16_BF16);
    if (st)
        return st;
    bool sym = (flags & W4A16_SYMMETRIC) != 0;
    if (!qpacked || !scales || !q_dev || !s_dev || (!sym && (!zeros || !z_dev)))
        return W4A16_ERR_NULL;
    st = check_weight_shape(N, K, g, flags);
    if (st)
        return st;
    if (!aligned16(qpacked) || !aligned16(scales) || !aligned16(q_dev) ||
        !aligned16(s_dev) || (!sym && (!aligned16(zeros) || !aligned16(z_dev))))
        return W4A16_ERR_ALIGN;
    return W4A16_OK;
}

int32_t w4a16_check_dequant_args(const uint32_t *qpacked, const uint16_t *scales,
                                 const uint32_t *zeros, int64_t N, int64_t K,
                                 int32_t g, uint32_t flags, const uint16_t *W) {
    int32_t st = check_flags(flags, W4A16_SYMMETRIC | W4A16_PARTIAL_LAST_GROUP | W4A16_BF16);
    if (st)
        return st;
    bool sym = (flags & W4A16_SYMMETRIC) != 0;
    if (!qpacked || !scales || !W || (!sym && !zeros))
        return W4A16_ERR_NULL;
    st = check_weight_shape(N, K, g, flags);
    if (st)
        return st;
    if (!aligned16(qpacked) || !aligned16(scales) || !aligned16(W) ||
        (!sym && !aligned16(zeros)))
        return W4A16_ERR_ALIGN;
    return W4A16_OK;
}

int32_t w4a16_check_quantize_args(const uint16_t *W, int64_t N, int64_t K, int32_t g,
                                  uint32_t flags, const uint32_t *qpacked,
                                  const uint16_t *scales, const uint32_t *zeros) {
    int32_t st = check_flags(flags, W4A16_SYMMETRIC | W4A16_PARTIAL_LAST_GROUP);
    if (st)
        return st;
    bool sym = (flags & W4A16_SYMMETRIC) != 0;
    if (!W || !qpacked || !scales || (!sym && !zeros))
        return W4A16_ERR_NULL;
    st = check_weight_shape(N, K, g, flags);
    if (st)
        return st;
    if (!aligned16(W) || !aligned16(qpacked) || !aligned16(scales) ||
        (!sym && !aligned16(zeros)))
        return W4A16_ERR_ALIGN;
    return W4A16_OK;
}

int32_t w4a16_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t g,
                                  uint32_t flags, size_t *bytes) {
    if (!bytes)
        return W4A16_ERR_NULL;
    int32_t st = check_flags(flags, W4A16_SYMMETRIC | W4A16_PARTIAL_LAST_GROUP | W4A16_BF16 |
                                        W4A16_PATH_SMALL_M | W4A16_PATH_LARGE_M);
    if (st)
        return st;
    if (M <= 0 || M > (int64_t(1) << 20))
        return W4A16_ERR_SHAPE;
    st = check_weight_shape(N, K, g, flags);
    if (st)
        return st;
    *bytes = plan_gemm(make_geom(M, N, K, g, flags), flags).ws_bytes;
    return W4A16_OK;
}

int32_t w4a16_gemm_kernel(int64_t M, int64_t N, int64_t K, int32_t g, uint32_t flags,
                          int32_t *path, int32_t *splits) {
    if (!path || !splits)
        return W4A16_ERR_NULL;
    int32_t st = check_flags(flags, W4A16_SYMMETRIC | W4A16_PARTIAL_LAST_GROUP | W4A16_BF16 |
                                        W4A16_PATH_SMALL_M | W4A16_PATH_LARGE_M);
    if (st)
        return st;
    if (M <= 0 || M > (int64_t(1) << 20))
        return W4A16_ERR_SHAPE;
    st = check_weight_shape(N, K, g, flags);
    if (st)
        return st;
    const GemmPlan p = plan_gemm(make_geom(M, N, K, g, flags), flags);
    *path = p.path == PATH_SMALL ? W4A16_KERNEL_SMALL_M : W4A16_KERNEL_LARGE_M;
    *splits = p.splits;
    return W4A16_OK;
}

int32_t w4a16_check_gemm_args(const uint16_t *X, int64_t M, int64_t K,
                              const void *q_dev, const void *s_dev,
                              const void *z_dev, int64_t N, int32_t g,
                              uint32_t flags, const uint16_t *Y,
                              const void *workspace, size_t workspace_bytes) {
    int32_t st = check_flags(flags, W4A16_SYMMETRIC | W4A16_PARTIAL_LAST_GROUP | W4A16_BF16 |
                                        W4A16_PATH_SMALL_M | W4A16_PATH_LARGE_M);
    if (st)
        return st;
    bool sym = (flags & W4A16_SYMMETRIC) != 0;
    if (!X || !q_dev || !s_dev || !Y || (!sym && !z_dev))
        return W4A16_ERR_NULL;
    if (M <= 0 || M > (int64_t(1) << 20) || M * K > (int64_t(1) << 34) ||
        M * N > (int64_t(1) << 34))
        return W4A16_ERR_SHAPE;
    st = check_weight_shape(N, K, g, flags);
    if (st)
        return st;
    if (!aligned16(X) || !aligned16(q_dev) || !aligned16(s_dev) || !aligned16(Y) ||
        (!sym && !aligned16(z_dev)))
        return W4A16_ERR_ALIGN;
    GemmPlan p = plan_gemm(make_geom(M, N, K, g, flags), flags);
    if (p.ws_bytes > 0) {
        if (!workspace)
            return W4A16_ERR_NULL;
        if (workspace_bytes < p.ws_bytes)
            return W4A16_ERR_WORKSPACE;
        if (!aligned16(workspace))
            return W4A16_ERR_ALIGN;
    }
    // X [M][K] and Y [M][N] must not overlap
    uintptr_t x0 = (uintptr_t)X, x1 = x0 + (uintptr_t)(M * K * 2);
    uintptr_t y0 = (uintptr_t)Y, y1 = y0 + (uintptr_t)(M * N * 2);
    if (x0 < y1 && y0 < x1)
        return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

}  // extern "C"
