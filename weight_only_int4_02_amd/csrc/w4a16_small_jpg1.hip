// Small-M kernel instances for 1 MFMA step(s) per group (g = 32), fp16.
#define W4A16_JPG 1
#define W4A16_BF 0
#include "w4a16_small_inst.inc"
