// fa_main_dropout.hip -- the dropout instantiations of the key-tile kernel of
// fa_main.hip, in a translation unit of their own so that they compile in
// parallel with the rest.
#define FA_TU_DROPOUT 1
#include "fa_main.hip"
