/*
 * qfa_probe — measurement helper of libqfa_probe.so, separate from the
 * attention library: the matrix-core throughput this GPU sustains for the
 * attention kernel's MFMA mix, with the clock it runs at. It computes
 * nothing the attention path uses.
 */
#ifndef QFA_PROBE_H
#define QFA_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * qfa_probe_mfma — launches `blocks` blocks of 4 waves (two blocks per CU,
 * the attention kernel's shape); each wave runs `iters` (a multiple of 4)
 * iterations of the MFMA
 * mix of one 32-row x 64-key attention tile on random operands:
 *   mix 0: 8 x v_mfma_i32_32x32x32_i8 + 16 x v_mfma_f32_32x32x16_bf16
 *          (2^20 multiply-adds x 2 = 2*2^20 ops per wave-iteration, half int8)
 *   mix 1: the 8 int8 MFMAs only;  mix 2: the 16 bf16 MFMAs only;
 *   mix 3: mix 0 plus the tile's softmax VALU work (per lane: 64 fma, 16 max,
 *          32 exp2, 16 bf16 pack, 16 dot2) on independent registers;
 *   mix 4: that VALU work alone.
 *   mix 5: mix 2 and mix 6: mix 0, on constant operands (codes 1, values 1.0);
 *   mix 7: the tile's MFMAs and its VALU work in separate phases between
 *          block barriers, blocks of 8 waves (blocks/2 launched, one per CU)
 *          whose second 4-wave group runs one phase behind the first (each
 *          SIMD then runs one wave's MFMA phase beside the other's VALU
 *          phase); mix 8: the same with both groups in step.
 *   sink then needs 512*ceil(blocks/2) floats;
 *   mix 9: mix 3 with the bf16 MFMAs' accumulators in AccVGPRs;
 *   mix 10: mix 3 with every accumulator in AccVGPRs.
 * Mixes 3 and 4 show how much of the VALU work the matrix-core time hides;
 * mixes 5 and 6 how much the operand data changes the sustained rate.
 * clocks: device buffer of 2*blocks uint64, written with (shader-clock
 *         cycles, 100 MHz reference ticks) of each block's loop.
 * sink:   device buffer of 256*blocks floats (keeps the results live).
 * Returns 0, or 1 for a bad argument, 3 for a launch error. Asynchronous on
 * `stream` (a hipStream_t).
 */
int qfa_probe_mfma(int blocks, int iters, int mix, unsigned long long* clocks, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QFA_PROBE_H */
