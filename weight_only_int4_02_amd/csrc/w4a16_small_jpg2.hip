// Small-M kernel instances for 2 MFMA step(s) per group (g = 64).
#define W4A16_JPG 2
#include "w4a16_small_inst.inc"
