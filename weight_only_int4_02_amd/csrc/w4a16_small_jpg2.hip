// Small-M kernel instances for 2 MFMA step(s) per group (g = 64), fp16.
#define W4A16_JPG 2
#define W4A16_BF 0
#include "w4a16_small_inst.inc"
