// Small-M kernel instances for 1 MFMA step(s) per group (g = 32), bfloat16.
#define W4A16_JPG 1
#define W4A16_BF 1
#include "w4a16_small_inst.inc"
